// Block-scaled NVFP4 GEMM for gfx950: Y[m][n] = g_x * g_w[n] * sum_k xq[m][k] * wq[n][k]
// where xq, wq are E2M1 codes times their E4M3 block scale.
//
// NVFP4 scales are E4M3 per 16 elements, which the gfx950 block-scaled FP4
// matrix instructions (power-of-two scales per 32 elements) cannot apply
// exactly.  Instead each operand is decoded exactly to FP16 in registers:
// code * scale has at most 6 significant bits and lies in [2^-10, 2688], so it
// is an exact normal FP16 value, and the FP16 matrix cores multiply exactly
// and accumulate in FP32.  The two global scales are applied once per output.
//
// K order inside one 128-element k-step: the matrix instruction sums over its
// K slots, so any assignment of K elements to slots works as long as both
// operands use the same one.  Lane groups take contiguous 32- or 64-element
// runs of the k-step (matching one 16-byte load), and each 8-element chunk a
// lane feeds to one instruction lies inside one 16-element block, so a lane
// applies exactly one block scale per chunk.
#include "common.h"

namespace nvfp4 {

__device__ __forceinline__ _Float16 scale_byte(uint32_t packed, int i) {
    return e4m3_to_f16((packed >> (8 * i)) & 0xFFu);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Skinny GEMM (M <= 16): one workgroup per 16 weight rows, 4 wavefronts split
// the k-steps and reduce through LDS.  16x16x32 FP16 instructions with the
// weight rows as the A operand and the (at most 16) tokens as B.
// ---------------------------------------------------------------------------
constexpr int kSkinnyM = 16;

__global__ __launch_bounds__(256) void gemm_skinny_kernel(int M, const uint8_t* __restrict__ a_codes,
                                                          const uint8_t* __restrict__ a_scales,
                                                          const float* __restrict__ g_x,
                                                          const uint8_t* __restrict__ w_codes,
                                                          const uint8_t* __restrict__ w_scales,
                                                          const float* __restrict__ colscale, int64_t N, int64_t K,
                                                          float* __restrict__ y, int64_t ld_y) {
    const int rb = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t KS = K / kPackK;
    const int r16 = lane & 15, kg = lane >> 4;
    const int tok = r16 < M ? r16 : M - 1;

    const uint8_t* wc = w_codes + (size_t)rb * KS * 1024 + kg * 256 + r16 * 16;
    const uint8_t* wsc = w_scales + (size_t)rb * KS * 128 + r16 * 8 + kg * 2;
    const uint8_t* xc = a_codes + (size_t)tok * (K / 2) + kg * 16;
    const uint8_t* xsc = a_scales + (size_t)tok * (K / 16) + kg * 2;

    float4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t ks = wave; ks < KS; ks += 4) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wc + ks * 1024);
        const uint32_t ws = *reinterpret_cast<const uint16_t*>(wsc + ks * 128);
        const uint4 xv = *reinterpret_cast<const uint4*>(xc + ks * 64);
        const uint32_t xs = *reinterpret_cast<const uint16_t*>(xsc + ks * 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const half8 a = decode8(word_of(wv, c), scale_byte(ws, c >> 1));
            const half8 b = decode8(word_of(xv, c), scale_byte(xs, c >> 1));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
        }
    }

    __shared__ float red[3][64][4];
    if (wave > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave - 1][lane][r] = acc[r];
    }
    __syncthreads();
    if (wave == 0) {
        const float gx = g_x[0];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = ((acc[r] + red[0][lane][r]) + red[1][lane][r]) + red[2][lane][r];
            const int64_t n = (int64_t)rb * 16 + (lane >> 4) * 4 + r;   // A row -> weight row
            if (r16 < M && n < N) y[(int64_t)r16 * ld_y + n] = s * (gx * colscale[n]);
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled GEMM: 128x128 output tile per workgroup, 2x2 wavefronts of 64x64, each
// a 2x2 grid of 32x32x16 FP16 instructions.  Operands load straight from
// global memory into registers (activations row-major, weights pre-swizzled).
// ---------------------------------------------------------------------------
constexpr int kTileM = 128, kTileN = 128;

__global__ __launch_bounds__(256) void gemm_tile_kernel(int64_t M, const uint8_t* __restrict__ a_codes,
                                                        const uint8_t* __restrict__ a_scales,
                                                        const float* __restrict__ g_x,
                                                        const uint8_t* __restrict__ w_codes,
                                                        const uint8_t* __restrict__ w_scales,
                                                        const float* __restrict__ colscale, int64_t N, int64_t K,
                                                        float* __restrict__ y, int64_t ld_y) {
    const int64_t tn = blockIdx.x, tm = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KS = K / kPackK;

    const uint8_t* ac[2];
    const uint8_t* as[2];
    const uint8_t* bc[2];
    const uint8_t* bs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t m = tm * kTileM + wm * 64 + i * 32 + l32;
        if (m >= M) m = M - 1;
        ac[i] = a_codes + m * (K / 2) + h * 32;
        as[i] = a_scales + m * (K / 16) + h * 4;
        const int64_t n = tn * kTileN + wn * 64 + i * 32 + l32;
        bc[i] = w_codes + (size_t)(n >> 4) * KS * 1024 + (2 * h) * 256 + (n & 15) * 16;
        bs[i] = w_scales + (size_t)(n >> 4) * KS * 128 + (n & 15) * 8 + h * 4;
    }

    float16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int64_t ks = 0; ks < KS; ++ks) {
        uint4 alo[2], ahi[2], blo[2], bhi[2];
        uint32_t asc[2], bsc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            alo[i] = *reinterpret_cast<const uint4*>(ac[i] + ks * 64);
            ahi[i] = *reinterpret_cast<const uint4*>(ac[i] + ks * 64 + 16);
            asc[i] = *reinterpret_cast<const uint32_t*>(as[i] + ks * 8);
            blo[i] = *reinterpret_cast<const uint4*>(bc[i] + ks * 1024);
            bhi[i] = *reinterpret_cast<const uint4*>(bc[i] + ks * 1024 + 256);
            bsc[i] = *reinterpret_cast<const uint32_t*>(bs[i] + ks * 128);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            half8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t aw = c < 4 ? word_of(alo[i], c) : word_of(ahi[i], c - 4);
                const uint32_t bw = c < 4 ? word_of(blo[i], c) : word_of(bhi[i], c - 4);
                a[i] = decode8(aw, scale_byte(asc[i], c >> 1));
                b[i] = decode8(bw, scale_byte(bsc[i], c >> 1));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    const float gx = g_x[0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = tn * kTileN + wn * 64 + j * 32 + l32;
        if (n >= N) continue;
        const float cs = gx * colscale[n];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = tm * kTileM + wm * 64 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                if (m < M) y[m * ld_y + n] = acc[i][j][r] * cs;
            }
        }
    }
}

size_t gemm_workspace_bytes(int64_t, const nvfp4_weight_desc&) { return 0; }

hipError_t launch_gemm(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                       const nvfp4_weight_desc& d, float* y, int64_t ld_y, void*, size_t, hipStream_t stream) {
    const uint8_t* blob = static_cast<const uint8_t*>(d.blob);
    const uint8_t* wc = blob + d.codes_offset;
    const uint8_t* wsc = blob + d.scales_offset;
    const float* cs = reinterpret_cast<const float*>(blob + d.colscale_offset);
    if (M <= kSkinnyM) {
        hipLaunchKernelGGL(gemm_skinny_kernel, dim3((unsigned)(d.n_padded / 16)), dim3(256), 0, stream,
                           (int)M, a_codes, a_scales, g_x, wc, wsc, cs, d.n, d.k, y, ld_y);
    } else {
        dim3 grid((unsigned)(d.n_padded / kTileN), (unsigned)((M + kTileM - 1) / kTileM));
        hipLaunchKernelGGL(gemm_tile_kernel, grid, dim3(256), 0, stream, M, a_codes, a_scales, g_x, wc, wsc, cs,
                           d.n, d.k, y, ld_y);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
