// Weight packing: canonical NVFP4 sub-modules -> one blob in MFMA operand order.
//
// Blob layout (all offsets from the blob start; n_pad = n rounded up to 256):
//   [0, 256)          header: magic, version, n, k, n_pad, n_modules
//   codes_offset      codes, 16-byte units ordered [n/16][k/128][kg 0..3][row%16]:
//                     unit (rb, ks, kg, r) = bytes [ks*64 + kg*16, +16) of row rb*16+r,
//                     i.e. elements [ks*128 + kg*32, +32) of that row.  A wavefront
//                     reading 64 consecutive units fetches 1 KB contiguous, and each
//                     lane holds exactly the 32 K-elements it feeds to the matrix cores.
//   scales_offset     scales, 8-byte units ordered [n/16][k/128][row%16]:
//                     unit (rb, ks, r) = the 8 block scales of row rb*16+r in k-step ks.
//   colscale_offset   FP32 [n_pad]: the global scale of the module that owns each row
//                     (0 for padding rows), so a fused projection keeps every
//                     sub-module's own scale ("Why Gated DeltaNet Survives 4-Bit
//                     Quantization", section "Critical Lessons for Model Serving").
// Padding rows have code 0 and scale 0, so they contribute exact zeros.
#include "common.h"

namespace nvfp4 {

struct PackArgs {
    const uint8_t* codes[NVFP4_MAX_MODULES];
    const uint8_t* scales[NVFP4_MAX_MODULES];
    const float* g_w[NVFP4_MAX_MODULES];
    int64_t row_off[NVFP4_MAX_MODULES + 1];
    int32_t n_modules;
    int64_t n, n_pad, k;
    uint8_t* blob;
    size_t codes_off, scales_off, colscale_off;
};

__device__ __forceinline__ int module_of(const PackArgs& a, int64_t row) {
    int s = 0;
    while (s + 1 < a.n_modules && row >= a.row_off[s + 1]) ++s;
    return s;
}

__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
    const int64_t KS = a.k / kPackK;
    const int64_t n_code_units = a.n_pad * a.k / 32;     // 16-byte units
    const int64_t n_scale_units = a.n_pad * KS;          // 8-byte units
    const int64_t total = n_code_units + n_scale_units + a.n_pad;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        if (i < n_code_units) {
            const int64_t r = i & 15, kg = (i >> 4) & 3, rest = i >> 6;
            const int64_t ks = rest % KS, rb = rest / KS;
            const int64_t row = rb * kPackRows + r;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < a.n) {
                const int s = module_of(a, row);
                const uint8_t* src = a.codes[s] + (row - a.row_off[s]) * (a.k / 2) + ks * 64 + kg * 16;
                v = *reinterpret_cast<const uint4*>(src);
            }
            *reinterpret_cast<uint4*>(a.blob + a.codes_off + i * 16) = v;
        } else if (i < n_code_units + n_scale_units) {
            const int64_t j = i - n_code_units;
            const int64_t r = j & 15, rest = j >> 4;
            const int64_t ks = rest % KS, rb = rest / KS;
            const int64_t row = rb * kPackRows + r;
            uint2 v = make_uint2(0, 0);
            if (row < a.n) {
                const int s = module_of(a, row);
                const uint8_t* src = a.scales[s] + (row - a.row_off[s]) * (a.k / 16) + ks * 8;
                v = *reinterpret_cast<const uint2*>(src);
            }
            *reinterpret_cast<uint2*>(a.blob + a.scales_off + j * 8) = v;
        } else {
            const int64_t row = i - n_code_units - n_scale_units;
            float c = 0.0f;
            if (row < a.n) c = a.g_w[module_of(a, row)][0];
            reinterpret_cast<float*>(a.blob + a.colscale_off)[row] = c;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        uint32_t* h32 = reinterpret_cast<uint32_t*>(a.blob);
        int64_t* h64 = reinterpret_cast<int64_t*>(a.blob + 8);
        h32[0] = NVFP4_WEIGHT_MAGIC;
        h32[1] = NVFP4_WEIGHT_VERSION;
        h64[0] = a.n;
        h64[1] = a.k;
        h64[2] = a.n_pad;
        h64[3] = a.n_modules;
    }
}

struct UnpackArgs {
    const uint8_t* blob;
    size_t codes_off, scales_off, colscale_off;
    int64_t n, k;
    uint8_t* codes;
    uint8_t* scales;
    float* colscale;
};

__global__ __launch_bounds__(256) void unpack_kernel(UnpackArgs a) {
    const int64_t KS = a.k / kPackK;
    const int64_t n_code_units = a.n * a.k / 32;
    const int64_t n_scale_units = a.n * KS;
    const int64_t total = n_code_units + n_scale_units + a.n;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        if (i < n_code_units) {
            // canonical unit i: row, 16-byte column chunk
            const int64_t row = i / (a.k / 32), chunk = i % (a.k / 32);
            const int64_t ks = chunk / 4, kg = chunk % 4;
            const int64_t rb = row / kPackRows, r = row % kPackRows;
            const int64_t u = ((rb * KS + ks) * 4 + kg) * 16 + r;
            *reinterpret_cast<uint4*>(a.codes + i * 16) =
                *reinterpret_cast<const uint4*>(a.blob + a.codes_off + u * 16);
        } else if (i < n_code_units + n_scale_units) {
            const int64_t j = i - n_code_units;
            const int64_t row = j / KS, ks = j % KS;
            const int64_t rb = row / kPackRows, r = row % kPackRows;
            const int64_t u = (rb * KS + ks) * 16 + r;
            *reinterpret_cast<uint2*>(a.scales + j * 8) =
                *reinterpret_cast<const uint2*>(a.blob + a.scales_off + u * 8);
        } else {
            const int64_t row = i - n_code_units - n_scale_units;
            a.colscale[row] = reinterpret_cast<const float*>(a.blob + a.colscale_off)[row];
        }
    }
}

static int grid_for(int64_t total) {
    int64_t g = (total + 255) / 256;
    if (g > 8192) g = 8192;
    return (int)(g < 1 ? 1 : g);
}

hipError_t launch_pack(const nvfp4_weight_desc& d, const uint8_t* const* codes, const uint8_t* const* scales,
                       const float* const* g_w, uint8_t* blob, hipStream_t stream) {
    PackArgs a = {};
    for (int s = 0; s < d.n_modules; ++s) {
        a.codes[s] = codes[s];
        a.scales[s] = scales[s];
        a.g_w[s] = g_w[s];
        a.row_off[s] = d.module_row_offset[s];
    }
    a.row_off[d.n_modules] = d.n;
    a.n_modules = d.n_modules;
    a.n = d.n;
    a.n_pad = d.n_padded;
    a.k = d.k;
    a.blob = blob;
    a.codes_off = d.codes_offset;
    a.scales_off = d.scales_offset;
    a.colscale_off = d.colscale_offset;
    const int64_t total = a.n_pad * a.k / 32 + a.n_pad * (a.k / kPackK) + a.n_pad;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_unpack(const nvfp4_weight_desc& d, uint8_t* codes, uint8_t* scales, float* colscale,
                         hipStream_t stream) {
    UnpackArgs a = {};
    a.blob = static_cast<const uint8_t*>(d.blob);
    a.codes_off = d.codes_offset;
    a.scales_off = d.scales_offset;
    a.colscale_off = d.colscale_offset;
    a.n = d.n;
    a.k = d.k;
    a.codes = codes;
    a.scales = scales;
    a.colscale = colscale;
    const int64_t total = a.n * a.k / 32 + a.n * (a.k / kPackK) + a.n;
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(total)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
