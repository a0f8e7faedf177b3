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
constexpr size_t kBlobHeader = 256;

// ---------------------------------------------------------------------------
// Encodings (IEEE FP32 decisions, no fused operations).
// ---------------------------------------------------------------------------

// Non-negative finite u -> E4M3 byte, nearest value, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float u) {
    if (u >= kE4M3Max) return 0x7Eu;
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

// Two FP32 values -> one byte of E2M1 codes (first value in the low nibble).
// The gfx950 conversion with a unit scale rounds to nearest with ties to the
// even code, saturates at 6 and keeps the sign bit of values that round to 0;
// that is the encoding rule used throughout, bit for bit.
__device__ __forceinline__ uint32_t e2m1_pair(float lo, float hi) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, lo, hi, 1.0f, 0) & 0xFFu;
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
// Host launchers (each returns hipSuccess or the launch error).
// ---------------------------------------------------------------------------

int quantize_partials_count(int64_t rows, int64_t K);
hipError_t launch_quantize(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x,
                           uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                           float* partials, int n_partials, hipStream_t stream);

hipError_t launch_pack(const nvfp4_weight_desc& d, const uint8_t* const* codes,
                       const uint8_t* const* scales, const float* const* g_w, uint8_t* blob,
                       hipStream_t stream);
hipError_t launch_unpack(const nvfp4_weight_desc& d, uint8_t* codes, uint8_t* scales, float* colscale,
                         hipStream_t stream);

size_t gemm_workspace_bytes(int64_t M, const nvfp4_weight_desc& d);
hipError_t launch_gemm(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                       const nvfp4_weight_desc& d, float* y, int64_t ld_y, void* ws, size_t ws_bytes,
                       hipStream_t stream);

}  // namespace nvfp4
