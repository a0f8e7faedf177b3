// Host side of the C ABI declared in include/nvfp4.h: argument validation (before
// any HIP call), descriptor construction, device check and kernel dispatch.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>

#include "common.h"

namespace {

thread_local std::string t_last_error;

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    t_last_error = buf;
    return st;
}

nvfp4_status ok() {
    t_last_error.clear();
    return NVFP4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

nvfp4_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(NVFP4_ERR_NO_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
    }
    int state = dev < 64 ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
    if (state == 0) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(NVFP4_ERR_NO_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
        }
        state = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        if (dev < 64) g_arch_ok[dev].store(state, std::memory_order_relaxed);
        if (state == 2) return fail(NVFP4_ERR_NO_DEVICE, "device %d is %s, this library is built for gfx950", dev, p.gcnArchName);
    }
    if (state == 2) return fail(NVFP4_ERR_NO_DEVICE, "device %d is not a gfx950", dev);
    return NVFP4_OK;
}

nvfp4_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Layout of a packed blob for the given shape (see pack.hip).
bool blob_layout(int n_modules, const int64_t* rows, int64_t K, nvfp4_weight_desc* d) {
    if (n_modules < 1 || n_modules > NVFP4_MAX_MODULES || rows == nullptr || K <= 0 || K % nvfp4::kPackK != 0)
        return false;
    std::memset(d, 0, sizeof(*d));
    int64_t n = 0;
    for (int s = 0; s < n_modules; ++s) {
        if (rows[s] < 1 || rows[s] > (int64_t(1) << 40)) return false;
        d->module_rows[s] = rows[s];
        d->module_row_offset[s] = n;
        n += rows[s];
    }
    if (K > (int64_t(1) << 30) || n > (int64_t(1) << 40)) return false;
    d->magic = NVFP4_WEIGHT_MAGIC;
    d->version = NVFP4_WEIGHT_VERSION;
    d->n = n;
    d->k = K;
    d->n_padded = round_up(n, nvfp4::kPackNAlign);
    if (d->n_padded * K / 2 > nvfp4::kMaxCodeBytes) return false;   // kernels address codes with 32-bit offsets
    d->n_modules = n_modules;
    d->codes_offset = nvfp4::kBlobHeader;
    d->scales_offset = d->codes_offset + (size_t)(d->n_padded * K / 2);
    d->colscale_offset = (size_t)round_up((int64_t)(d->scales_offset + (size_t)(d->n_padded * K / 16)), 256);
    d->blob_bytes = d->colscale_offset + (size_t)d->n_padded * sizeof(float);
    return true;
}

nvfp4_status check_desc(const nvfp4_weight_desc* w) {
    if (w == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "weight descriptor is NULL");
    if (w->magic != NVFP4_WEIGHT_MAGIC || w->version != NVFP4_WEIGHT_VERSION)
        return fail(NVFP4_ERR_DESCRIPTOR, "weight descriptor magic/version mismatch (0x%08x v%u)", w->magic, w->version);
    nvfp4_weight_desc ref;
    if (!blob_layout(w->n_modules, w->module_rows, w->k, &ref))
        return fail(NVFP4_ERR_DESCRIPTOR, "weight descriptor has an invalid shape");
    if (ref.n != w->n || ref.n_padded != w->n_padded || ref.codes_offset != w->codes_offset ||
        ref.scales_offset != w->scales_offset || ref.colscale_offset != w->colscale_offset ||
        ref.blob_bytes != w->blob_bytes)
        return fail(NVFP4_ERR_DESCRIPTOR, "weight descriptor fields are inconsistent");
    for (int s = 0; s < w->n_modules; ++s)
        if (ref.module_row_offset[s] != w->module_row_offset[s])
            return fail(NVFP4_ERR_DESCRIPTOR, "weight descriptor module offsets are inconsistent");
    if (w->blob == nullptr || !aligned(w->blob, 256)) return fail(NVFP4_ERR_DESCRIPTOR, "weight blob is NULL or not 256-byte aligned");
    return NVFP4_OK;
}

// ---------------------------------------------------------------------------
// Scratch for nvfp4_linear_noalloc: the workspace of nvfp4_linear (the few-token
// kernel's counters, then the quantizer's amax partials) in a device array
// of the library, so that entry point allocates nothing.  Each GPU holds its own
// copy; host code reaches it only through the address hipGetSymbolAddress
// returns on that device (the array's name is a host-side stand-in).
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = 81920;   // every shape's workspace fits (at most 2048 + 73728 + 4096)
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void clear_scratch_kernel(uint32_t* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // per device, once set up

// Device address of the current device's scratch, set up (address looked up,
// contents cleared by a kernel on `stream`) on the first call on that device.
nvfp4_status scratch_for_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return fail(NVFP4_ERR_NO_DEVICE, "no usable HIP device for the static scratch");
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return fail(NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        hipLaunchKernelGGL(clear_scratch_kernel, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                           (int)(kNoAllocScratchBytes / 4));
        e = hipGetLastError();
        if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_last_error(void) { return t_last_error.c_str(); }

nvfp4_status nvfp4_device_check(void) {
    nvfp4_status st = check_device();
    return st == NVFP4_OK ? ok() : st;
}

size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || K <= 0) return 0;
    return (size_t)round_up((int64_t)nvfp4::quantize_partials_count(rows, K) * (int64_t)sizeof(float), 256);
}

static nvfp4_status quantize_impl(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x, uint8_t* codes,
                                  uint8_t* scales, float* g, int g_mode, void* workspace, size_t workspace_bytes,
                                  void* stream, int rht, uint32_t signs) {
    if (rht && signs > 0xFFFFu) return fail(NVFP4_ERR_INVALID_ARG, "signs is a 16-bit mask (got 0x%x)", signs);
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown input dtype %d", in_dtype);
    if (g_mode != NVFP4_G_COMPUTE && g_mode != NVFP4_G_GIVEN)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown g mode %d", g_mode);
    if (g == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "g is NULL");
    if (rows < 0 || K <= 0 || K % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "need rows >= 0 and K > 0 a multiple of 16 (rows=%lld K=%lld)",
                    (long long)rows, (long long)K);
    if (ld_x < K) return fail(NVFP4_ERR_SHAPE, "ld_x (%lld) < K (%lld)", (long long)ld_x, (long long)K);
    if (rows > 0 && ld_x > INT64_MAX / rows) return fail(NVFP4_ERR_SHAPE, "tensor too large");
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (rows > 0) {
        if (x == nullptr || codes == nullptr || scales == nullptr)
            return fail(NVFP4_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
        if (!aligned(x, 16) || (ld_x * esize) % 16 != 0)
            return fail(NVFP4_ERR_UNSUPPORTED, "x must be 16-byte aligned with a 16-byte multiple row stride");
        if (!aligned(codes, 8)) return fail(NVFP4_ERR_UNSUPPORTED, "codes must be 8-byte aligned");
    }
    const int n_partials = nvfp4::quantize_partials_count(rows, K);
    if (g_mode == NVFP4_G_COMPUTE && rows > 0) {
        const size_t need = nvfp4_quantize_workspace_bytes(rows, K);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
            return fail(NVFP4_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    }
    nvfp4_status st = check_device();
    if (st != NVFP4_OK) return st;
    return launched(nvfp4::launch_quantize(x, in_dtype, rows, K, ld_x, codes, scales, g, g_mode,
                                           static_cast<float*>(workspace), n_partials,
                                           static_cast<hipStream_t>(stream), rht, signs),
                    "quantize launch");
}

nvfp4_status nvfp4_quantize(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x, uint8_t* codes,
                            uint8_t* scales, float* g, int g_mode, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return quantize_impl(x, in_dtype, rows, K, ld_x, codes, scales, g, g_mode, workspace, workspace_bytes, stream,
                         0, 0u);
}

nvfp4_status nvfp4_quantize_rht(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x, uint32_t signs,
                                uint8_t* codes, uint8_t* scales, float* g, int g_mode, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return quantize_impl(x, in_dtype, rows, K, ld_x, codes, scales, g, g_mode, workspace, workspace_bytes, stream,
                         1, signs);
}

static nvfp4_status quantize_t_impl(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                    uint8_t* codes, uint8_t* scales, float* g, int g_mode, void* workspace,
                                    size_t workspace_bytes, void* stream, int rht, uint32_t signs) {
    if (rht && signs > 0xFFFFu) return fail(NVFP4_ERR_INVALID_ARG, "signs is a 16-bit mask (got 0x%x)", signs);
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown input dtype %d", in_dtype);
    if (g_mode != NVFP4_G_COMPUTE && g_mode != NVFP4_G_GIVEN)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown g mode %d", g_mode);
    if (g == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "g is NULL");
    if (rows < 0 || cols < 0 || rows % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "need cols >= 0 and rows >= 0 a multiple of 16 (rows=%lld cols=%lld)",
                    (long long)rows, (long long)cols);
    if (ld_x < cols) return fail(NVFP4_ERR_SHAPE, "ld_x (%lld) < cols (%lld)", (long long)ld_x, (long long)cols);
    if (rows > 0 && ld_x > INT64_MAX / rows) return fail(NVFP4_ERR_SHAPE, "tensor too large");
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (rows > 0 && cols > 0) {
        if (x == nullptr || codes == nullptr || scales == nullptr)
            return fail(NVFP4_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
        if (!aligned(x, esize)) return fail(NVFP4_ERR_UNSUPPORTED, "x must be aligned to its element size");
        if (!aligned(codes, 8)) return fail(NVFP4_ERR_UNSUPPORTED, "codes must be 8-byte aligned");
    }
    const int n_partials = nvfp4::quantize_partials_count(rows, cols);
    if (g_mode == NVFP4_G_COMPUTE && rows > 0 && cols > 0) {
        const size_t need = nvfp4_quantize_workspace_bytes(rows, cols);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
            return fail(NVFP4_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    }
    nvfp4_status st = check_device();
    if (st != NVFP4_OK) return st;
    return launched(nvfp4::launch_quantize_t(x, in_dtype, rows, cols, ld_x, codes, scales, g, g_mode,
                                             static_cast<float*>(workspace), n_partials,
                                             static_cast<hipStream_t>(stream), rht, signs),
                    "quantize_t launch");
}

nvfp4_status nvfp4_quantize_t(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t* codes, uint8_t* scales, float* g, int g_mode, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return quantize_t_impl(x, in_dtype, rows, cols, ld_x, codes, scales, g, g_mode, workspace, workspace_bytes,
                           stream, 0, 0u);
}

nvfp4_status nvfp4_quantize_t_rht(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint32_t signs, uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return quantize_t_impl(x, in_dtype, rows, cols, ld_x, codes, scales, g, g_mode, workspace, workspace_bytes,
                           stream, 1, signs);
}

nvfp4_status nvfp4_quantize_both(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, float* g,
                                 int g_mode, void* workspace, size_t workspace_bytes, void* stream) {
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown input dtype %d", in_dtype);
    if (g_mode != NVFP4_G_COMPUTE && g_mode != NVFP4_G_GIVEN)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown g mode %d", g_mode);
    if (g == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "g is NULL");
    if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "need rows and cols >= 0, multiples of 16 (rows=%lld cols=%lld)",
                    (long long)rows, (long long)cols);
    if (ld_x < cols) return fail(NVFP4_ERR_SHAPE, "ld_x (%lld) < cols (%lld)", (long long)ld_x, (long long)cols);
    if (rows > 0 && ld_x > INT64_MAX / rows) return fail(NVFP4_ERR_SHAPE, "tensor too large");
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (rows > 0 && cols > 0) {
        if (x == nullptr || codes == nullptr || scales == nullptr || codes_t == nullptr || scales_t == nullptr)
            return fail(NVFP4_ERR_INVALID_ARG, "x and the four outputs must be non-NULL");
        if (!aligned(x, esize)) return fail(NVFP4_ERR_UNSUPPORTED, "x must be aligned to its element size");
        if (!aligned(codes, 4) || !aligned(codes_t, 8))
            return fail(NVFP4_ERR_UNSUPPORTED, "codes must be 4-byte and codes_t 8-byte aligned");
    }
    const int n_partials = nvfp4::quantize_partials_count(rows, cols);
    if (g_mode == NVFP4_G_COMPUTE && rows > 0 && cols > 0) {
        const size_t need = nvfp4_quantize_workspace_bytes(rows, cols);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
            return fail(NVFP4_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    }
    nvfp4_status st = check_device();
    if (st != NVFP4_OK) return st;
    return launched(nvfp4::launch_quantize_both(x, in_dtype, rows, cols, ld_x, codes, scales, codes_t, scales_t, g,
                                                g_mode, static_cast<float*>(workspace), n_partials,
                                                static_cast<hipStream_t>(stream)),
                    "quantize_both launch");
}

nvfp4_status nvfp4_kv_quantize_fp8(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                   uint8_t* codes, float* scale, int s_mode, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown input dtype %d", in_dtype);
    if (s_mode != NVFP4_G_COMPUTE && s_mode != NVFP4_G_GIVEN)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown scale mode %d", s_mode);
    if (scale == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "scale is NULL");
    if (rows < 0 || cols < 0)
        return fail(NVFP4_ERR_SHAPE, "need rows >= 0 and cols >= 0 (rows=%lld cols=%lld)", (long long)rows,
                    (long long)cols);
    if (ld_x < cols) return fail(NVFP4_ERR_SHAPE, "ld_x (%lld) < cols (%lld)", (long long)ld_x, (long long)cols);
    if (rows > 0 && (ld_x > INT64_MAX / rows || cols > INT64_MAX / rows)) return fail(NVFP4_ERR_SHAPE, "tensor too large");
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (rows > 0 && cols > 0) {
        if (x == nullptr || codes == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "x and codes must be non-NULL");
        if (!aligned(x, esize)) return fail(NVFP4_ERR_UNSUPPORTED, "x must be aligned to its element size");
    }
    const int n_partials = nvfp4::quantize_partials_count(rows, cols);
    if (s_mode == NVFP4_G_COMPUTE && rows > 0 && cols > 0) {
        const size_t need = nvfp4_quantize_workspace_bytes(rows, cols);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
            return fail(NVFP4_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    }
    nvfp4_status st = check_device();
    if (st != NVFP4_OK) return st;
    return launched(nvfp4::launch_kv_fp8(x, in_dtype, rows, cols, ld_x, codes, scale, s_mode,
                                         static_cast<float*>(workspace), n_partials,
                                         static_cast<hipStream_t>(stream)),
                    "kv fp8 launch");
}

size_t nvfp4_packed_weight_bytes(int n_modules, const int64_t* module_rows, int64_t K) {
    nvfp4_weight_desc d;
    if (!blob_layout(n_modules, module_rows, K, &d)) return 0;
    return d.blob_bytes;
}

nvfp4_status nvfp4_pack_weights(int n_modules, const int64_t* module_rows, int64_t K, const uint8_t* const* codes,
                                const uint8_t* const* scales, const float* const* g_w, void* blob, size_t blob_bytes,
                                nvfp4_weight_desc* desc_out, void* stream) {
    if (n_modules > NVFP4_MAX_MODULES)
        return fail(NVFP4_ERR_UNSUPPORTED, "at most %d modules per packed weight (got %d)", NVFP4_MAX_MODULES, n_modules);
    if (n_modules < 1) return fail(NVFP4_ERR_INVALID_ARG, "n_modules must be >= 1");
    if (module_rows == nullptr || codes == nullptr || scales == nullptr || g_w == nullptr || desc_out == nullptr)
        return fail(NVFP4_ERR_INVALID_ARG, "NULL array argument");
    for (int s = 0; s < n_modules; ++s)
        if (module_rows[s] < 1) return fail(NVFP4_ERR_SHAPE, "module %d has %lld rows", s, (long long)module_rows[s]);
    if (K <= 0 || K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K must be a positive multiple of 16 (got %lld)", (long long)K);
    if (K % nvfp4::kPackK != 0)
        return fail(NVFP4_ERR_UNSUPPORTED, "packed weights need K a multiple of %d (got %lld)", nvfp4::kPackK, (long long)K);
    nvfp4_weight_desc d;
    if (!blob_layout(n_modules, module_rows, K, &d)) return fail(NVFP4_ERR_SHAPE, "weight shape too large");
    for (int s = 0; s < n_modules; ++s) {
        if (codes[s] == nullptr || scales[s] == nullptr || g_w[s] == nullptr)
            return fail(NVFP4_ERR_INVALID_ARG, "module %d has a NULL codes/scales/g pointer", s);
        if (!aligned(codes[s], 16) || !aligned(scales[s], 8) || !aligned(g_w[s], 4))
            return fail(NVFP4_ERR_UNSUPPORTED, "module %d: codes must be 16-byte and scales 8-byte aligned", s);
    }
    if (blob == nullptr || !aligned(blob, 256)) return fail(NVFP4_ERR_INVALID_ARG, "blob must be non-NULL and 256-byte aligned");
    if (blob_bytes < d.blob_bytes)
        return fail(NVFP4_ERR_WORKSPACE, "blob needs %zu bytes (got %zu)", d.blob_bytes, blob_bytes);
    nvfp4_status st = check_device();
    if (st != NVFP4_OK) return st;
    d.blob = blob;
    hipError_t e = nvfp4::launch_pack(d, codes, scales, g_w, static_cast<uint8_t*>(blob), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "pack launch: %s", hipGetErrorString(e));
    *desc_out = d;
    return ok();
}

nvfp4_status nvfp4_pack_weights_train(const void* w, int in_dtype, int64_t n, int64_t k, int64_t ld_w, float* g,
                                      int g_mode, void* blob_fwd, size_t blob_fwd_bytes, nvfp4_weight_desc* desc_fwd,
                                      void* blob_bwd, size_t blob_bwd_bytes, nvfp4_weight_desc* desc_bwd,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown input dtype %d", in_dtype);
    if (g_mode != NVFP4_G_COMPUTE && g_mode != NVFP4_G_GIVEN)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown g mode %d", g_mode);
    if (w == nullptr || g == nullptr || desc_fwd == nullptr || desc_bwd == nullptr)
        return fail(NVFP4_ERR_INVALID_ARG, "w, g and both descriptors must be non-NULL");
    if (n <= 0 || k <= 0 || n % nvfp4::kPackK != 0 || k % nvfp4::kPackK != 0)
        return fail(NVFP4_ERR_SHAPE, "n and k must be positive multiples of %d (n=%lld k=%lld)", nvfp4::kPackK,
                    (long long)n, (long long)k);
    if (ld_w < k || ld_w > INT64_MAX / n) return fail(NVFP4_ERR_SHAPE, "bad ld_w (%lld)", (long long)ld_w);
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (!aligned(w, esize)) return fail(NVFP4_ERR_UNSUPPORTED, "w must be aligned to its element size");
    nvfp4_weight_desc df, db;
    if (!blob_layout(1, &n, k, &df) || !blob_layout(1, &k, n, &db)) return fail(NVFP4_ERR_SHAPE, "weight too large");
    if (blob_fwd == nullptr || blob_bwd == nullptr || !aligned(blob_fwd, 256) || !aligned(blob_bwd, 256))
        return fail(NVFP4_ERR_INVALID_ARG, "blobs must be non-NULL and 256-byte aligned");
    if (blob_fwd_bytes < df.blob_bytes || blob_bwd_bytes < db.blob_bytes)
        return fail(NVFP4_ERR_WORKSPACE, "blobs need %zu and %zu bytes (got %zu and %zu)", df.blob_bytes,
                    db.blob_bytes, blob_fwd_bytes, blob_bwd_bytes);
    const int n_partials = nvfp4::quantize_partials_count(n, k);
    if (g_mode == NVFP4_G_COMPUTE) {
        const size_t need = nvfp4_quantize_workspace_bytes(n, k);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 4))
            return fail(NVFP4_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    }
    nvfp4_status st = check_device();
    if (st != NVFP4_OK) return st;
    df.blob = blob_fwd;
    db.blob = blob_bwd;
    hipError_t e = nvfp4::launch_pack_train(w, in_dtype, n, k, ld_w, g, g_mode, static_cast<float*>(workspace),
                                            n_partials, df, db, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "pack_train launch: %s", hipGetErrorString(e));
    *desc_fwd = df;
    *desc_bwd = db;
    return ok();
}

nvfp4_status nvfp4_unpack_weights(const nvfp4_weight_desc* w, uint8_t* codes, uint8_t* scales, float* colscale,
                                  void* stream) {
    nvfp4_status st = check_desc(w);
    if (st != NVFP4_OK) return st;
    if (codes == nullptr || scales == nullptr || colscale == nullptr)
        return fail(NVFP4_ERR_INVALID_ARG, "unpack outputs must be non-NULL");
    if (!aligned(codes, 16) || !aligned(scales, 8) || !aligned(colscale, 4))
        return fail(NVFP4_ERR_UNSUPPORTED, "unpack: codes must be 16-byte and scales 8-byte aligned");
    st = check_device();
    if (st != NVFP4_OK) return st;
    return launched(nvfp4::launch_unpack(*w, codes, scales, colscale, static_cast<hipStream_t>(stream)), "unpack launch");
}

size_t nvfp4_gemm_workspace_bytes(int64_t M, const nvfp4_weight_desc* w) {
    if (w == nullptr || M < 0) return 0;
    return nvfp4::gemm_workspace_bytes(M, *w);
}

static nvfp4_status gemm_impl(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                              const nvfp4_weight_desc* w, const nvfp4::Epilogue& gp, void* y, int64_t ld_y,
                              void* workspace, size_t workspace_bytes, void* stream) {
    nvfp4_status st = check_desc(w);
    if (st != NVFP4_OK) return st;
    if (M < 0) return fail(NVFP4_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
    if (M == 0) return ok();
    if (a_codes == nullptr || a_scales == nullptr || g_x == nullptr || y == nullptr)
        return fail(NVFP4_ERR_INVALID_ARG, "a_codes, a_scales, g_x and y must be non-NULL");
    if (ld_y < w->n) return fail(NVFP4_ERR_SHAPE, "ld_y (%lld) < n (%lld)", (long long)ld_y, (long long)w->n);
    if (M > (int64_t(1) << 31) || ld_y > INT64_MAX / M) return fail(NVFP4_ERR_SHAPE, "M too large");
    if (M * w->k / 2 > nvfp4::kMaxCodeBytes)
        return fail(NVFP4_ERR_UNSUPPORTED, "activation codes above 2 GiB (M*K/2 = %lld)", (long long)(M * w->k / 2));
    if (!aligned(a_codes, 16) || !aligned(a_scales, 4) || !aligned(y, gp.out_bf16 ? 2 : 4))
        return fail(NVFP4_ERR_UNSUPPORTED, "a_codes must be 16-byte, a_scales 4-byte and y element aligned");
    const size_t need = nvfp4::gemm_workspace_bytes(M, *w);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(NVFP4_ERR_WORKSPACE, "gemm workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    st = check_device();
    if (st != NVFP4_OK) return st;
    return launched(nvfp4::launch_gemm(M, a_codes, a_scales, g_x, *w, static_cast<float*>(y), ld_y, workspace,
                                       workspace_bytes, gp, static_cast<hipStream_t>(stream)),
                    "gemm launch");
}

// Gate parameters -> the kernels' form, after checking them against the weight.
static nvfp4_status gate_params(const nvfp4_gdn_gates* g, const nvfp4_weight_desc* w, nvfp4::Epilogue& gp) {
    if (g == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "gates is NULL");
    if (w == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "w is NULL");
    if (g->n_a < 0 || g->n_b < 0 || g->a_col < 0 || g->b_col < 0 || g->a_col > w->n - g->n_a ||
        g->b_col > w->n - g->n_b)
        return fail(NVFP4_ERR_SHAPE, "gate columns [%lld, +%lld) and [%lld, +%lld) must lie inside [0, %lld)",
                    (long long)g->a_col, (long long)g->n_a, (long long)g->b_col, (long long)g->n_b, (long long)w->n);
    if (g->n_a > 0 && g->n_b > 0 && g->a_col < g->b_col + g->n_b && g->b_col < g->a_col + g->n_a)
        return fail(NVFP4_ERR_SHAPE, "decay and write-strength columns overlap");
    if (g->n_a > 0 && (g->a_log == nullptr || g->dt_bias == nullptr))
        return fail(NVFP4_ERR_INVALID_ARG, "a_log and dt_bias must be non-NULL when n_a > 0");
    if (g->n_a > 0 && (!aligned(g->a_log, 4) || !aligned(g->dt_bias, 4)))
        return fail(NVFP4_ERR_UNSUPPORTED, "a_log and dt_bias must be 4-byte aligned");
    gp.a_col = (int32_t)g->a_col;   // < w->n < 2^31 (a packed weight holds at most 2 GiB of codes)
    gp.n_a = (int32_t)g->n_a;
    gp.b_col = (int32_t)g->b_col;
    gp.n_b = (int32_t)g->n_b;
    gp.a_log = g->a_log;
    gp.dt_bias = g->dt_bias;
    return NVFP4_OK;
}

nvfp4_status nvfp4_gemm(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                        const nvfp4_weight_desc* w, float* y, int64_t ld_y, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return gemm_impl(M, a_codes, a_scales, g_x, w, nvfp4::Epilogue{}, y, ld_y, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_gemm_gated(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                              const nvfp4_weight_desc* w, const nvfp4_gdn_gates* gates, float* y, int64_t ld_y,
                              void* workspace, size_t workspace_bytes, void* stream) {
    nvfp4_status st = check_desc(w);
    if (st != NVFP4_OK) return st;
    nvfp4::Epilogue gp;
    st = gate_params(gates, w, gp);
    if (st != NVFP4_OK) return st;
    return gemm_impl(M, a_codes, a_scales, g_x, w, gp, y, ld_y, workspace, workspace_bytes, stream);
}

// The counters of the one-launch few-token path come first, reserved for every
// M, so that the amax partials of the two-launch path (quantize, then the
// product) never land on them: one workspace may serve calls with any M.
// The few-token kernel's part of the workspace (flags, then its copy of the
// activation encoding), reserved whatever M is, so that one workspace serves
// calls with any token count; the quantizer's partial maxima follow it.
static size_t linear_counter_bytes(int64_t, const nvfp4_weight_desc& w) {
    return std::max(nvfp4::kSkinnyCounterBytes, nvfp4::skinny_workspace_bytes(w));
}

size_t nvfp4_linear_workspace_bytes(int64_t M, int in_dtype, const nvfp4_weight_desc* w) {
    if (w == nullptr || M < 0 || w->k <= 0 || w->n_padded <= 0) return 0;
    (void)in_dtype;
    return linear_counter_bytes(M, *w) + nvfp4_quantize_workspace_bytes(M, w->k);
}

// use_static: the workspace is the library's static scratch (nvfp4_linear_noalloc),
// looked up after the arguments are validated and a device is present.
static nvfp4_status linear_impl(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                                uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w,
                                const nvfp4::Epilogue& gp, void* y_out, int64_t ld_y, void* workspace,
                                size_t workspace_bytes, void* stream, bool use_static = false) {
    float* y = static_cast<float*>(y_out);   // bf16 storage when gp.out_bf16 (the kernels store through store_y)
    nvfp4_status st = check_desc(w);
    if (st != NVFP4_OK) return st;
    const int64_t K = w->k;
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown input dtype %d", in_dtype);
    if (g_mode != NVFP4_G_COMPUTE && g_mode != NVFP4_G_GIVEN)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown g mode %d", g_mode);
    if (M < 0) return fail(NVFP4_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
    if (g_x == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "g_x is NULL");
    if (ld_x < K) return fail(NVFP4_ERR_SHAPE, "ld_x (%lld) < K (%lld)", (long long)ld_x, (long long)K);
    if (M > 0) {
        if (x == nullptr || x_codes == nullptr || x_scales == nullptr || y == nullptr)
            return fail(NVFP4_ERR_INVALID_ARG, "x, x_codes, x_scales and y must be non-NULL");
        if (ld_y < w->n) return fail(NVFP4_ERR_SHAPE, "ld_y (%lld) < n (%lld)", (long long)ld_y, (long long)w->n);
        if (M > (int64_t(1) << 31) || ld_x > INT64_MAX / M || ld_y > INT64_MAX / M)
            return fail(NVFP4_ERR_SHAPE, "M too large");
        if (M * K / 2 > nvfp4::kMaxCodeBytes)
            return fail(NVFP4_ERR_UNSUPPORTED, "activation codes above 2 GiB (M*K/2 = %lld)", (long long)(M * K / 2));
        const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
        if (!aligned(x, 16) || (ld_x * esize) % 16 != 0)
            return fail(NVFP4_ERR_UNSUPPORTED, "x must be 16-byte aligned with a 16-byte multiple row stride");
        if (!aligned(x_codes, 16) || !aligned(x_scales, 4) || !aligned(y, gp.out_bf16 ? 2 : 4))
            return fail(NVFP4_ERR_UNSUPPORTED, "x_codes must be 16-byte, x_scales 4-byte and y element aligned");
    }
    const size_t need = nvfp4_linear_workspace_bytes(M, in_dtype, w);
    if (use_static) {
        if (need > kNoAllocScratchBytes)
            return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_linear_noalloc: this shape needs %zu bytes of scratch, above "
                        "the library's static %zu bytes; use nvfp4_linear with a workspace", need,
                        kNoAllocScratchBytes);
    } else if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))) {
        return fail(NVFP4_ERR_WORKSPACE, "linear workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    }
    st = check_device();
    if (st != NVFP4_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (use_static) {
        st = scratch_for_current_device(s, &workspace);
        if (st != NVFP4_OK) return st;
        workspace_bytes = kNoAllocScratchBytes;
    }
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    // the fused few-token kernel addresses the activations with 32-bit offsets
    const int64_t esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const bool skinny = nvfp4::skinny_applies(M, *w);
    const bool fused = skinny && M * ld_x * esize <= INT32_MAX;
    const size_t counter_bytes = linear_counter_bytes(M, *w);   // the counters come first
    float* partials = reinterpret_cast<float*>(wsb + counter_bytes);
    const int n_partials = nvfp4::quantize_partials_count(M, K);
    if (M == 0 || !fused) {
        hipError_t e = nvfp4::launch_quantize(x, in_dtype, M, K, ld_x, x_codes, x_scales, g_x, g_mode, partials,
                                              n_partials, s);
        if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "linear quantize launch: %s", hipGetErrorString(e));
        if (M == 0) return ok();
        return launched(nvfp4::launch_gemm(M, x_codes, x_scales, g_x, *w, y, ld_y, nullptr, 0, gp, s),
                        "linear gemm launch");
    }
    return launched(nvfp4::launch_skinny(M, x, in_dtype, ld_x, g_x, g_mode, x_codes, x_scales, true, *w, y, ld_y,
                                         workspace, gp, s),
                    "linear launch");
}

nvfp4_status nvfp4_linear(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes, uint8_t* x_scales,
                          float* g_x, int g_mode, const nvfp4_weight_desc* w, float* y, int64_t ld_y,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return linear_impl(x, in_dtype, M, ld_x, x_codes, x_scales, g_x, g_mode, w, nvfp4::Epilogue{}, y, ld_y,
                       workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_linear_noalloc(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                                  uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w, float* y,
                                  int64_t ld_y, void* stream) {
    return linear_impl(x, in_dtype, M, ld_x, x_codes, x_scales, g_x, g_mode, w, nvfp4::Epilogue{}, y, ld_y, nullptr,
                       0, stream, true);
}

// Epilogue descriptor -> the kernels' form.
static nvfp4_status epilogue(const nvfp4_epilogue* ep, const nvfp4_weight_desc* w, nvfp4::Epilogue& out) {
    if (ep == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "epilogue is NULL");
    if (ep->y_dtype != NVFP4_OUT_F32 && ep->y_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_ERR_INVALID_ARG, "unknown output dtype %d", ep->y_dtype);
    if (ep->reserved != 0) return fail(NVFP4_ERR_INVALID_ARG, "epilogue.reserved must be 0");
    nvfp4_status st = check_desc(w);
    if (st != NVFP4_OK) return st;
    if (ep->gates != nullptr) {
        st = gate_params(ep->gates, w, out);
        if (st != NVFP4_OK) return st;
    }
    out.out_bf16 = ep->y_dtype == NVFP4_OUT_BF16;
    return NVFP4_OK;
}

nvfp4_status nvfp4_gemm_ex(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                           const nvfp4_weight_desc* w, const nvfp4_epilogue* ep, void* y, int64_t ld_y,
                           void* workspace, size_t workspace_bytes, void* stream) {
    nvfp4::Epilogue e;
    nvfp4_status st = epilogue(ep, w, e);
    if (st != NVFP4_OK) return st;
    return gemm_impl(M, a_codes, a_scales, g_x, w, e, y, ld_y, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_linear_ex(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                             uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w,
                             const nvfp4_epilogue* ep, void* y, int64_t ld_y, void* workspace,
                             size_t workspace_bytes, void* stream) {
    nvfp4::Epilogue e;
    nvfp4_status st = epilogue(ep, w, e);
    if (st != NVFP4_OK) return st;
    return linear_impl(x, in_dtype, M, ld_x, x_codes, x_scales, g_x, g_mode, w, e, y, ld_y, workspace,
                       workspace_bytes, stream);
}

nvfp4_status nvfp4_linear_gated(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                                uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w,
                                const nvfp4_gdn_gates* gates, float* y, int64_t ld_y, void* workspace,
                                size_t workspace_bytes, void* stream) {
    nvfp4_status st = check_desc(w);
    if (st != NVFP4_OK) return st;
    nvfp4::Epilogue gp;
    st = gate_params(gates, w, gp);
    if (st != NVFP4_OK) return st;
    return linear_impl(x, in_dtype, M, ld_x, x_codes, x_scales, g_x, g_mode, w, gp, y, ld_y, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
