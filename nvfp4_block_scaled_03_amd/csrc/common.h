// Internal declarations shared by the HIP translation units of libnvfp4.
// Device helpers for the NVFP4 encodings (E2M1 element codes, E4M3 block
// scales) and the host-side launch entry points of each kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "nvfp4.h"

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Largest E2M1 magnitude and largest finite E4M3 value; their product maps a
// tensor's amax onto code 6 of a block scaled by 448.
constexpr float kE2M1Max = 6.0f;
constexpr float kE4M3Max = 448.0f;
constexpr float kGlobalRange = kE2M1Max * kE4M3Max;  // 2688
constexpr float kGFloor = 7.8886090522101181e-31f;   // 2^-100

// Geometry of the packed weight blob (see pack.hip).
constexpr int kPackRows = 16;      // rows per packed row-block
constexpr int kPackK = 128;        // K elements per packed k-step (64 code bytes per row)
constexpr int kPackNAlign = 256;   // n is padded to a multiple of this
constexpr int64_t kMaxCodeBytes = int64_t(1) << 31;   // per operand: the GEMMs use 32-bit byte offsets
constexpr size_t kBlobHeader = 256;

constexpr int kComputeUnits = 256;   // MI355X: the work splits are sized for this many
// Few-token products: at most 16 tokens (one 16-column matrix-instruction tile).
constexpr int kSkinnyM = 16;
constexpr int kMaxAmaxPartials = 1024;   // upper bound of quantize_partials_count

// ---------------------------------------------------------------------------
// Encodings (IEEE FP32 decisions, no fused operations).
// ---------------------------------------------------------------------------

// Non-negative u -> E4M3 byte, nearest value, ties to even, saturating at 448.
// Infinity (a block amax times a caller's very large 1/g) and the NaN that
// div6 makes of it saturate too.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float u) {
    if (!(u < kE4M3Max)) return 0x7Eu;
    if (u < 0.015625f) {                              // below 2^-6: subnormal grid m * 2^-9
        return (uint32_t)__builtin_rintf(u * 512.0f); // exact scaling, RNE to 0..8 (8 = 2^-6)
    }
    uint32_t b = __float_as_uint(u);
    b += 0x7FFFFu + ((b >> 20) & 1u);                 // RNE to 3 mantissa bits
    uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
    return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 byte (0..0x7E) -> FP32 value (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t s) {
    uint32_t e = s >> 3, m = s & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// E4M3 byte -> FP16 (exact).  Placing the 7 magnitude bits at FP16 bits 13..7
// gives S * 2^-8 (FP16 subnormal for E4M3 subnormals); scaling by 2^8 is exact.
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t s) {
    uint16_t bits = (uint16_t)((s & 0x7Fu) << 7);
    return __builtin_bit_cast(_Float16, bits) * (_Float16)256.0f;
}

// 8 E2M1 codes (one 32-bit word, element 2j in the low nibble of byte j) times
// one FP16 block scale -> 8 FP16 values.  code * scale has at most 6 significant
// bits and lies in [2^-10, 2688], so every product is an exact normal FP16.
__device__ __forceinline__ half8 decode8(uint32_t w, _Float16 s) {
    half2v s2 = {s, s};
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    half8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

// ---------------------------------------------------------------------------
// Quantizer building blocks (IEEE FP32, one rounding per operation; every
// translation unit that encodes is compiled with FP contraction off).
// ---------------------------------------------------------------------------

// 8 consecutive elements -> FP32 (bf16 widens exactly).
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
// The same as streaming loads (nontemporal: the lines are not kept in the
// caches), for passes that read each byte once.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
    const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(q.x, q.y, q.z, q.w);
}
__device__ __forceinline__ void load8_stream(const uint16_t* p, float v[8]) {
    const uint4 u = load16_stream(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8_stream(const float* p, float v[8]) {
    const uint4 a = load16_stream(p), b = load16_stream(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One 16-element block of raw input, as loaded (two or four 16-byte vectors).
template <typename T> struct RawBlock;
template <> struct RawBlock<uint16_t> { uint4 v[2]; };
template <> struct RawBlock<float> { uint4 v[4]; };

__device__ __forceinline__ void widen(const RawBlock<uint16_t>& r, float v[16]) {
    load8(reinterpret_cast<const uint16_t*>(&r.v[0]), v);
    load8(reinterpret_cast<const uint16_t*>(&r.v[1]), v + 8);
}
__device__ __forceinline__ void widen(const RawBlock<float>& r, float v[16]) {
    load8(reinterpret_cast<const float*>(&r.v[0]), v);
    load8(reinterpret_cast<const float*>(&r.v[2]), v + 8);
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    return m;
}

template <int kThreads>
__device__ __forceinline__ float block_max(float m) {
    __shared__ float red[kThreads / 64];
    m = wave_max(m);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wid] = m;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// g from the tensor amax: fl32(amax/2688); 1 for an all-zero tensor; floored at 2^-100.
__device__ __forceinline__ float global_scale_from_amax(float amax) {
    if (amax == 0.0f) return 1.0f;
    float g = amax / kGlobalRange;
    return g < kGFloor ? kGFloor : g;
}

// fl32(t / 6) for t >= 0 without a division: q0 = fl32(t * fl32(1/6)), the
// exact remainder t - 6*q0 by one fused multiply-add, and one more to correct
// q0.  For every finite t >= 2^-124 this is the correctly rounded quotient
// (all 2^31 non-negative floats checked on the CPU); below that the quotient
// lies under 2^-126, far below the smallest nonzero E4M3 scale, so the scale
// it leads to (0) is the same either way.
__device__ __forceinline__ float div6(float t) {
    const float c = 1.0f / 6.0f;
    const float q0 = t * c;
    const float r = __builtin_fmaf(-q0, 6.0f, t);
    return __builtin_fmaf(r, c, q0);
}

// r = fl32(s_enc / S) for every scale byte S (0 for S = 0): 128 entries, one
// correctly rounded division each, shared by all the blocks of a workgroup.
// Threads tid, tid + nthreads, ... fill it; the caller synchronises before use.
__device__ __forceinline__ void fill_recip_table(float* tab, float s_enc, int tid, int nthreads) {
    for (int i = tid; i < 128; i += nthreads) tab[i] = (i == 0 || i > 0x7E) ? 0.0f : s_enc / e4m3_to_f32((uint32_t)i);
}

// max |v| over one 16-element block.
__device__ __forceinline__ float block_amax(const float v[16]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, __builtin_fabsf(v[i]));
    return m;
}

// Randomized Hadamard transform of one 16-element block, in place:
// v <- H16 . D . v / 4, D the diagonal of the sign mask (bit i negates element
// i), H16 the Hadamard matrix in natural order.  The negation is a sign-bit
// flip (exact); the butterflies run in the stage order h = 1, 2, 4, 8 with one
// FP32 rounding per addition, since codes are bit-exact and that order is part
// of the definition; the product by 1/4 is exact above the subnormal range.
__device__ __forceinline__ void rht16(float v[16], uint32_t signs) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((signs >> i) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (!(i & h)) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= 0.25f;
}

// Encode one 16-element block held in v[16], whose max |v| is bamax, with the
// tensor's s_enc and its table of s_enc / S (or, with rtab == nullptr, that
// entry divided out here: the same correctly rounded quotient).
__device__ __forceinline__ void encode_block(const float v[16], float bamax, float s_enc, const float* rtab,
                                             uint32_t& lo, uint32_t& hi, uint32_t& scale) {
    const float t = bamax * s_enc;
    const uint32_t S = e4m3_rne_sat(div6(t));
    const float r = rtab ? rtab[S] : (S == 0 ? 0.0f : s_enc / e4m3_to_f32(S));
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = v[i] * r;
    // Two elements per conversion, first in the low nibble; each writes one byte
    // of the word and keeps the other three.  The gfx950 conversion with a unit
    // scale rounds to nearest with ties to the even code, saturates at 6 and
    // keeps the sign of values that round to 0: the encoding rule, bit for bit.
    uint32_t a = 0, b = 0;
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[0], q[1], 1.0f, 0);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[2], q[3], 1.0f, 1);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[4], q[5], 1.0f, 2);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[6], q[7], 1.0f, 3);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[8], q[9], 1.0f, 0);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[10], q[11], 1.0f, 1);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[12], q[13], 1.0f, 2);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[14], q[15], 1.0f, 3);
    lo = a;
    hi = b;
    scale = S;
}

// ---------------------------------------------------------------------------
// Operand loads and decode for the GEMMs.
// ---------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A buffer offset past every record count used here (they are all <= INT32_MAX):
// a load from it returns zero, with no branch around the load.
constexpr uint32_t kOutOfBounds = 0xFFFFFF00u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ _Float16 scale_byte(uint32_t packed, int i) {
    return e4m3_to_f16((packed >> (8 * i)) & 0xFFu);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Host launchers (each returns hipSuccess or the launch error).
// ---------------------------------------------------------------------------

int quantize_partials_count(int64_t rows, int64_t K);
// Per-workgroup partial maxima of |x| (n_partials workgroups), as the first kernel of the quantizer.
hipError_t launch_quantize_both(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, float* g,
                                int g_mode, float* partials, int n_partials, hipStream_t stream);
// Both packed operands of one training weight (forward: rows x cols along cols;
// backward: its transpose), from one read; the descriptors are filled in.
hipError_t launch_pack_train(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x, float* g,
                             int g_mode, float* partials, int n_partials, const nvfp4_weight_desc& df,
                             const nvfp4_weight_desc& db, hipStream_t stream);
hipError_t launch_kv_fp8(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                         float* scale, int s_mode, float* partials, int n_partials, hipStream_t stream);

// rht != 0: every block goes through rht16 with the given sign mask first.
hipError_t launch_quantize(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x,
                           uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                           float* partials, int n_partials, hipStream_t stream, int rht = 0, uint32_t signs = 0);
hipError_t launch_quantize_t(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t* codes, uint8_t* scales, float* g, int g_mode, float* partials, int n_partials,
                             hipStream_t stream, int rht = 0, uint32_t signs = 0);

hipError_t launch_pack(const nvfp4_weight_desc& d, const uint8_t* const* codes,
                       const uint8_t* const* scales, const float* const* g_w, uint8_t* blob,
                       hipStream_t stream);
hipError_t launch_unpack(const nvfp4_weight_desc& d, uint8_t* codes, uint8_t* scales, float* colscale,
                         hipStream_t stream);

// Gate epilogue of a fused Gated DeltaNet projection (anthology-of-the-sota
// record theory-128, Kozyrev and Maiboroda 2026, section "The account", the
// paragraph on the gates' parameterization): output columns [a_col, a_col + n_a) become the state
// decay exp(-exp(A) * softplus(y + bias)) of their head, columns
// [b_col, b_col + n_b) the write strength sigmoid(y).  The kernels take it as a
// compile-time option, so products without gates carry none of it.
struct Epilogue {
    int32_t a_col = 0, n_a = 0, b_col = 0, n_b = 0;   // columns fit 31 bits (the packed weight is <= 2 GiB)
    const float* a_log = nullptr;
    const float* dt_bias = nullptr;
    int32_t out_bf16 = 0;                             // Y as bf16 (round to nearest even) instead of FP32
};

// FP32 -> bf16 bits, round to nearest with ties to even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32) under the default rounding mode, one operation.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// One output element: FP32, or bf16 when the epilogue asks for it (y then
// points at bf16 storage and idx counts bf16 elements).
__device__ __forceinline__ void store_y(float* y, int64_t idx, float v, const Epilogue& ep) {
    if (ep.out_bf16)
        reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
    else
        y[idx] = v;
}

// Whether any column of [n0, n1) is a gate column (wave-uniform when n0, n1 are).
__device__ __forceinline__ bool gates_touch(int64_t n0, int64_t n1, const Epilogue& gp) {
    return (gp.n_a > 0 && n0 < gp.a_col + gp.n_a && gp.a_col < n1) ||
           (gp.n_b > 0 && n0 < gp.b_col + gp.n_b && gp.b_col < n1);
}

// The gate of one output column: what it is and its per-head parameters, read
// once per column (the store loops then run without loads): kind 1 = decay
// with bias and c = exp(A), kind 2 = write strength, 0 = no gate.
struct GateCol {
    int kind;
    float bias, c;
};

__device__ __forceinline__ GateCol gate_col(int64_t n, const Epilogue& gp) {
    const uint32_t ha = (uint32_t)((int32_t)n - gp.a_col), hb = (uint32_t)((int32_t)n - gp.b_col);
    if (ha < (uint32_t)gp.n_a) return GateCol{1, gp.dt_bias[ha], expf(gp.a_log[ha])};
    if (hb < (uint32_t)gp.n_b) return GateCol{2, 0.0f, 0.0f};
    return GateCol{0, 0.0f, 0.0f};
}

// FP32, with softplus and the sigmoid in forms that cannot overflow and without
// divergent branches (a lane's rows mix signs, so branches would run both sides):
// softplus(z) = max(z, 0) + log1p(exp(-|z|)) and sigmoid(y) = (y >= 0 ? 1 : e) / (1 + e)
// with e = exp(-|y|), each the same operations as the two-sided forms.
__device__ __forceinline__ float gate_apply(float y, const GateCol& g) {
    if (g.kind == 1) {
        const float z = y + g.bias;
        const float sp = (z > 0.0f ? z : 0.0f) + log1pf(expf(-__builtin_fabsf(z)));
        return expf(-(g.c * sp));
    }
    if (g.kind == 2) {
        const float e = expf(-__builtin_fabsf(y));
        return (y >= 0.0f ? 1.0f : e) / (1.0f + e);
    }
    return y;
}

__device__ __forceinline__ float gate(float y, int64_t n, const Epilogue& gp) { return gate_apply(y, gate_col(n, gp)); }

size_t gemm_workspace_bytes(int64_t M, const nvfp4_weight_desc& d);
hipError_t launch_gemm(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                       const nvfp4_weight_desc& d, float* y, int64_t ld_y, void* ws, size_t ws_bytes,
                       const Epilogue& gp, hipStream_t stream);

// Few-token products (skinny.hip).  With the activations encoded in the same
// launch (nvfp4_linear) the workspace holds 256 bytes of launch-tagged flags
// per XCD (zero before the first use; no launch needs them reset).  The
// product alone needs none.
constexpr size_t kSkinnyCounterBytes = 2048;
bool skinny_applies(int64_t M, const nvfp4_weight_desc& d);
size_t skinny_workspace_bytes(const nvfp4_weight_desc& d);
hipError_t launch_skinny(int64_t M, const void* x, int in_dtype, int64_t ld_x, float* g_x, int g_mode,
                         uint8_t* x_codes, uint8_t* x_scales, bool quantize, const nvfp4_weight_desc& d, float* y,
                         int64_t ld_y, void* ws, const Epilogue& gp, hipStream_t stream);

}  // namespace nvfp4
