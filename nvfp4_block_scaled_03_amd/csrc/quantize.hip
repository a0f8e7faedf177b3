// NVFP4 activation/weight quantizer for gfx950.
//
// Two kernels, because the per-tensor scale is a global dependency of every
// block's encoding:
//   1. amax_partials: each workgroup reduces max|x| over its share of the tensor
//      and writes one partial (no atomics, no initialised memory needed).
//   2. encode: every workgroup reduces the partials itself (a few KB from L2),
//      derives g and s_enc = fl32(1/g), and encodes 16-element blocks along K:
//      bamax -> E4M3 scale of fl32(fl32(bamax*s_enc)/6) -> r = fl32(s_enc/S)
//      (from a 128-entry table per workgroup)
//      -> E2M1 code of fl32(x*r) per element -> two codes per byte.
// The block structure and per-tensor scale follow "Why Gated DeltaNet Survives
// 4-Bit Quantization" (sections "Why the 'Fragile' Recurrence is Actually
// Robust" and "Critical Lessons for Model Serving").  Every decision is taken
// in IEEE FP32 with one rounding per operation (contraction disabled below),
// so codes and scales are bit-for-bit reproducible.
#include "common.h"

#pragma clang fp contract(off)

namespace nvfp4 {

constexpr int kQThreads = 256;
constexpr int kMaxPartials = kMaxAmaxPartials;

// Segments of a row: each thread reads kSegVec vectors of 8 elements.
constexpr int kSegVec = 4;
constexpr int64_t kSegElems = (int64_t)kQThreads * 8 * kSegVec;

__device__ __forceinline__ float elem_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float elem_f32(float v) { return v; }

template <typename T>
__global__ __launch_bounds__(kQThreads) void amax_partials_kernel(const T* __restrict__ x, int64_t rows, int64_t K,
                                                                  int64_t ld, float* __restrict__ partials,
                                                                  int vec = 1) {
    // A contiguous tensor is one long row.
    if (ld == K) { K = rows * K; rows = 1; ld = K; }
    const int64_t seg_per_row = (K + kSegElems - 1) / kSegElems;
    const int64_t nseg = rows * seg_per_row;
    float m = 0.0f;
    for (int64_t s = blockIdx.x; s < nseg; s += gridDim.x) {
        const int64_t r = s / seg_per_row;
        const int64_t c0 = (s - r * seg_per_row) * kSegElems;
        const T* row = x + r * ld;
#pragma unroll
        for (int u = 0; u < kSegVec; ++u) {
            const int64_t c = c0 + ((int64_t)u * kQThreads + threadIdx.x) * 8;
            if (vec && c + 8 <= K) {
                float v[8];
                load8(row + c, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[i]));
            } else if (c < K) {          // x^T encoding only: row tails, or rows not 16-byte aligned
                const int64_t e = c + 8 < K ? c + 8 : K;
                for (int64_t i = c; i < e; ++i) m = fmaxf(m, __builtin_fabsf(elem_f32(row[i])));
            }
        }
    }
    m = block_max<kQThreads>(m);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Per-workgroup max |v| over transformed blocks (the global amax of the
// transformed tensor), one partial per workgroup, blocks by grid stride.
template <typename T>
__global__ __launch_bounds__(kQThreads) void amax_rht_kernel(const T* __restrict__ x, int64_t rows, int64_t K,
                                                             int64_t ld, uint32_t signs, float* __restrict__ partials) {
    const int64_t bpr = K / 16, nblk = rows * bpr;
    float m = 0.0f;
    for (int64_t b = (int64_t)blockIdx.x * kQThreads + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * kQThreads) {
        const int64_t r = b / bpr;
        const T* src = x + r * ld + (b - r * bpr) * 16;
        float v[16];
        load8(src, v);
        load8(src + 8, v + 8);
        rht16(v, signs);
        m = fmaxf(m, block_amax(v));
    }
    m = block_max<kQThreads>(m);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

template <typename T, bool RHT>
__global__ __launch_bounds__(kQThreads) void encode_kernel(const T* __restrict__ x, int64_t rows, int64_t K, int64_t ld,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                           float* __restrict__ g_io, int g_given,
                                                           const float* __restrict__ partials, int n_partials,
                                                           uint32_t signs) {
    __shared__ float s_senc;
    __shared__ float rtab[128];
    if (g_given) {
        if (threadIdx.x == 0) s_senc = 1.0f / g_io[0];
        __syncthreads();
    } else {
        float m = 0.0f;
        for (int i = threadIdx.x; i < n_partials; i += kQThreads) m = fmaxf(m, partials[i]);
        m = block_max<kQThreads>(m);
        if (threadIdx.x == 0) {
            const float g = global_scale_from_amax(m);
            s_senc = 1.0f / g;
            if (blockIdx.x == 0) g_io[0] = g;
        }
        __syncthreads();
    }
    const float s_enc = s_senc;
    fill_recip_table(rtab, s_enc, threadIdx.x, kQThreads);
    __syncthreads();
    const int64_t bpr = K / 16;                 // blocks per row
    const int64_t nblk = rows * bpr;
    const bool dense = (ld == K);
    for (int64_t b = (int64_t)blockIdx.x * kQThreads + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * kQThreads) {
        const T* src;
        if (dense) {
            src = x + b * 16;
        } else {
            const int64_t r = b / bpr;
            src = x + r * ld + (b - r * bpr) * 16;
        }
        float v[16];
        load8(src, v);
        load8(src + 8, v + 8);
        if (RHT) rht16(v, signs);
        uint32_t lo, hi, S;
        encode_block(v, block_amax(v), s_enc, rtab, lo, hi, S);
        *reinterpret_cast<uint2*>(codes + b * 8) = make_uint2(lo, hi);
        scales[b] = (uint8_t)S;
    }
}

__global__ void write_unit_g_kernel(float* g) { g[0] = 1.0f; }

// ---------------------------------------------------------------------------
// FP8 (E4M3) KV-cache quantizer with one FP32 scale s per tensor (calibrated
// and given, or calibrated on the tensor: s = fl32(amax / 448), 1 for an
// all-zero tensor, floored at 2^-100).  Per element, like the NVFP4 element
// step: q = fl32(x * fl32(1/s)), byte = sign of q | nearest E4M3 magnitude
// (ties to even, saturating at 448); NaN gives 0x7F with its sign.  Each
// thread converts runs of 8 elements of a row (one 16-byte or two 16-byte
// loads, one 8-byte store); ragged or unaligned runs go element by element.
// ---------------------------------------------------------------------------
constexpr float kKvRange = 448.0f;

__device__ __forceinline__ uint32_t kv_byte(float v, float r) {
    const float q = v * r;
    const float a = __builtin_fabsf(q);
    const uint32_t mag = a != a ? 0x7Fu : e4m3_rne_sat(a);
    return ((__float_as_uint(q) >> 24) & 0x80u) | mag;
}

template <typename T>
__global__ __launch_bounds__(kQThreads) void kv_fp8_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                           int64_t ld, uint8_t* __restrict__ codes,
                                                           float* __restrict__ s_io, int s_given,
                                                           const float* __restrict__ partials, int n_partials,
                                                           int vec) {
    __shared__ float s_r;
    if (s_given) {
        if (threadIdx.x == 0) s_r = 1.0f / s_io[0];
    } else {
        float m = 0.0f;
        for (int i = threadIdx.x; i < n_partials; i += kQThreads) m = fmaxf(m, partials[i]);
        m = block_max<kQThreads>(m);
        if (threadIdx.x == 0) {
            float sc = m / kKvRange;
            sc = m == 0.0f ? 1.0f : (sc < kGFloor ? kGFloor : sc);
            s_r = 1.0f / sc;
            if (blockIdx.x == 0) s_io[0] = sc;
        }
    }
    __syncthreads();
    const float r = s_r;
    const int64_t runs_per_row = (cols + 7) / 8, nruns = rows * runs_per_row;
    for (int64_t u = (int64_t)blockIdx.x * kQThreads + threadIdx.x; u < nruns; u += (int64_t)gridDim.x * kQThreads) {
        const int64_t row = u / runs_per_row, col = (u - row * runs_per_row) * 8;
        const T* src = x + row * ld + col;
        uint8_t* dst = codes + row * cols + col;
        if (vec && col + 8 <= cols) {
            float v[8];
            load8(src, v);
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w0 |= kv_byte(v[i], r) << (8 * i);
                w1 |= kv_byte(v[4 + i], r) << (8 * i);
            }
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        } else {
            const int64_t e = col + 8 <= cols ? 8 : cols - col;
            for (int64_t i = 0; i < e; ++i) dst[i] = (uint8_t)kv_byte(elem_f32(src[i]), r);
        }
    }
}

// ---------------------------------------------------------------------------
// The encoding of x^T (blocks of 16 consecutive rows of x, one output row per
// column of x): the other operand orientation of the training GEMMs
// (dX = dY.W needs W quantized along its rows, dW = dY^T.X needs dY and X
// quantized along their rows).  Same global scale (the amax is the same), same
// block rule.
//
// No LDS: each lane loads a 16-row x 16-byte patch of x (16 row vectors, all
// in flight at once), which holds kVec whole blocks of x^T, one per column,
// and encodes them from its registers.  A wavefront is 8 row groups x 8
// column lanes, so each load instruction reads eight 128-byte row segments;
// a workgroup of 4 wavefronts covers 512 rows x 8*kVec columns and writes,
// per output row, 256 consecutive code bytes (two cache lines, merged in L2
// from the 32 lanes that share the column).  Narrower segments measured
// faster than 256- or 512-byte ones.
// ---------------------------------------------------------------------------
constexpr int kTLanesC = 8;                 // lanes across columns (128-byte row segments)
constexpr int kTRows = 4 * (64 / kTLanesC) * 16;   // rows per workgroup tile (512)

// MODE: kTEncode (plain), kTEncodeRht (transformed blocks), kTAmaxRht (no
// encoding: max |v| of the transformed blocks, one partial per workgroup into
// amax_out, tiles by grid stride), kTBoth (plain, and from the same registers
// the row encoding too: a row block of 16 columns spans 16/kVec neighbouring
// lanes, which combine their maxima by lane exchange and each encode their own
// kVec elements; needs cols % 16 == 0).
enum { kTEncode = 0, kTEncodeRht = 1, kTAmaxRht = 2, kTBoth = 3 };

// The row-block part of a lane's patch: NE (8 or 4) elements of one row whose
// 16-element block has max |v| = bamax; the same operations as encode_block.
template <int NE>
__device__ __forceinline__ uint32_t encode_part(const float* v, float bamax, float s_enc, const float* rtab,
                                                uint32_t& scale) {
    const uint32_t S = e4m3_rne_sat(div6(bamax * s_enc));
    const float r = rtab[S];
    uint32_t a = 0;
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[0] * r, v[1] * r, 1.0f, 0);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[2] * r, v[3] * r, 1.0f, 1);
    if constexpr (NE == 8) {
        a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[4] * r, v[5] * r, 1.0f, 2);
        a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[6] * r, v[7] * r, 1.0f, 3);
    }
    scale = S;
    return a;
}

template <typename T, int MODE>
__global__ __launch_bounds__(kQThreads) void encode_t_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                             int64_t ld, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, float* __restrict__ g_io,
                                                             int g_given, const float* __restrict__ partials,
                                                             int n_partials, int vec, uint32_t signs,
                                                             float* __restrict__ amax_out,
                                                             uint8_t* __restrict__ codes_r = nullptr,
                                                             uint8_t* __restrict__ scales_r = nullptr) {
    __shared__ float s_senc;
    __shared__ float rtab[128];
    float s_enc = 0.0f, m = 0.0f;
    if (MODE != kTAmaxRht) {
        if (g_given) {
            if (threadIdx.x == 0) s_senc = 1.0f / g_io[0];
        } else {
            float pm = 0.0f;
            for (int i = threadIdx.x; i < n_partials; i += kQThreads) pm = fmaxf(pm, partials[i]);
            pm = block_max<kQThreads>(pm);
            if (threadIdx.x == 0) {
                const float g = global_scale_from_amax(pm);
                s_senc = 1.0f / g;
                if (blockIdx.x == 0) g_io[0] = g;
            }
        }
        __syncthreads();
        s_enc = s_senc;
        fill_recip_table(rtab, s_enc, threadIdx.x, kQThreads);
        __syncthreads();
    }

    constexpr int kVec = 16 / (int)sizeof(T);                 // columns per lane (one 16-byte vector)
    constexpr int kRG = 64 / kTLanesC;                         // row groups per wavefront
    constexpr int kTCols = kTLanesC * kVec;
    const int64_t tiles_r = (rows + kTRows - 1) / kTRows, tiles_c = (cols + kTCols - 1) / kTCols;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cl = lane % kTLanesC, rg = lane / kTLanesC;
    for (int64_t tile_id = blockIdx.x; tile_id < tiles_r * tiles_c; tile_id += gridDim.x) {
        // column-major tile order: workgroups launched together finish whole output rows
        // (measured faster than row-major or grouped orders, whose reads are more sequential)
        const int64_t tr = tile_id % tiles_r, tc = tile_id / tiles_r;
        const int64_t r0 = tr * kTRows + (w * kRG + rg) * 16;       // this lane's 16 rows
        const int64_t c0 = tc * kTCols + (int64_t)kVec * cl;        // and kVec columns
        if (r0 >= rows || c0 >= cols) continue;
        const T* src = x + r0 * ld + c0;
        T e[16][kVec];
        if (vec && c0 + kVec <= cols) {
#pragma unroll
            for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(e[i]) = *reinterpret_cast<const uint4*>(src + i * ld);
        } else {                                 // ragged last columns or unaligned rows
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int k = 0; k < kVec; ++k) e[i][k] = c0 + k < cols ? src[i * ld + k] : T(0);
        }
        if constexpr (MODE == kTBoth) {
            // row blocks: lanes cl, cl ^ 1 (and cl ^ 2 for FP32) hold one 16-column block of each row
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v[kVec];
                float pm = 0.0f;
#pragma unroll
                for (int k = 0; k < kVec; ++k) {
                    v[k] = elem_f32(e[i][k]);
                    pm = fmaxf(pm, __builtin_fabsf(v[k]));
                }
                pm = fmaxf(pm, __shfl_xor(pm, 1, 64));
                if constexpr (kVec == 4) pm = fmaxf(pm, __shfl_xor(pm, 2, 64));
                uint32_t sc;
                const uint32_t w = encode_part<kVec>(v, pm, s_enc, rtab, sc);
                uint8_t* crow = codes_r + (r0 + i) * (cols / 2) + c0 / 2;
                if constexpr (kVec == 8)
                    *reinterpret_cast<uint32_t*>(crow) = w;
                else
                    *reinterpret_cast<uint16_t*>(crow) = (uint16_t)w;
                if ((c0 & 15) == 0) scales_r[(r0 + i) * (cols / 16) + c0 / 16] = (uint8_t)sc;
            }
        }
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            if (c0 + k >= cols) break;
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = elem_f32(e[i][k]);
            if (MODE == kTEncodeRht || MODE == kTAmaxRht) rht16(v, signs);
            if (MODE == kTAmaxRht) {
                m = fmaxf(m, block_amax(v));
                continue;
            }
            uint32_t lo, hi, sc;
            encode_block(v, block_amax(v), s_enc, rtab, lo, hi, sc);
            *reinterpret_cast<uint2*>(codes + (c0 + k) * (rows / 2) + r0 / 2) = make_uint2(lo, hi);
            scales[(c0 + k) * (rows / 16) + r0 / 16] = (uint8_t)sc;
        }
    }
    if (MODE == kTAmaxRht) {
        m = block_max<kQThreads>(m);
        if (threadIdx.x == 0) amax_out[blockIdx.x] = m;
    }
}

// Small tensors (at most kSmallThreads * P blocks) in one launch: every one of
// the P workgroups loads the whole tensor (thread t holds blocks t, t + 1024,
// ...), reduces max|x| itself, so no workgroup depends on another, and then
// encodes its own share: workgroup w encodes the w-th block of every thread.
constexpr int kSmallThreads = 1024;

template <typename T, int P>
__global__ __launch_bounds__(kSmallThreads) void quantize_small_kernel(const T* __restrict__ x, int64_t rows,
                                                                       int64_t K, int64_t ld,
                                                                       uint8_t* __restrict__ codes,
                                                                       uint8_t* __restrict__ scales,
                                                                       float* __restrict__ g_io, int g_given) {
    const int bpr = (int)(K / 16);
    const int nblk = (int)rows * bpr;
    const rsrc_t rx = make_rsrc(x, (uint64_t)rows * ld * sizeof(T));
    RawBlock<T> raw[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {   // branch-free: blocks past the tensor read as zero
        const int b = threadIdx.x + i * kSmallThreads;
        const int r = b / bpr, kb = b - r * bpr;
        const uint32_t off = b < nblk ? (uint32_t)(((int64_t)r * ld + (int64_t)kb * 16) * (int64_t)sizeof(T))
                                      : kOutOfBounds;
#pragma unroll
        for (int q = 0; q < (int)(sizeof(RawBlock<T>) / 16); ++q) raw[i].v[q] = bload16(rx, off, (uint32_t)q * 16);
    }
    float g;
    if (g_given) {
        g = g_io[0];
    } else {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            float v[16];
            widen(raw[i], v);
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, __builtin_fabsf(v[e]));
        }
        g = global_scale_from_amax(block_max<kSmallThreads>(m));
        if (blockIdx.x == 0 && threadIdx.x == 0) g_io[0] = g;
    }
    RawBlock<T> mine = raw[0];
#pragma unroll
    for (int i = 1; i < P; ++i)
        if ((int)blockIdx.x == i) mine = raw[i];
    __shared__ float rtab[128];
    const float s_enc = 1.0f / g;
    fill_recip_table(rtab, s_enc, threadIdx.x, kSmallThreads);
    __syncthreads();
    const int b = threadIdx.x + (int)blockIdx.x * kSmallThreads;
    if (b < nblk) {
        float v[16];
        widen(mine, v);
        uint32_t lo, hi, S;
        encode_block(v, block_amax(v), s_enc, rtab, lo, hi, S);
        *reinterpret_cast<uint2*>(codes + (int64_t)b * 8) = make_uint2(lo, hi);
        scales[b] = (uint8_t)S;
    }
}

// Blocks per thread of the one-launch path for this tensor, or 0 when it does not apply.
static int small_blocks_per_thread(int64_t rows, int64_t K, int64_t ld, int in_dtype) {
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const int64_t nblk = rows * (K / 16);
    const int max_p = in_dtype == NVFP4_IN_BF16 ? 8 : 4;   // raw registers: 8 or 16 per block
    if (rows < 1 || nblk > (int64_t)kSmallThreads * max_p || rows * ld * esize > INT32_MAX) return 0;
    return (int)((nblk + kSmallThreads - 1) / kSmallThreads);
}

template <typename T>
static hipError_t launch_small(int p, const T* x, int64_t rows, int64_t K, int64_t ld, uint8_t* codes,
                               uint8_t* scales, float* g, int given, hipStream_t stream) {
#define NVFP4_QS(P)                                                                                             \
    case P:                                                                                                     \
        hipLaunchKernelGGL((quantize_small_kernel<T, P>), dim3(P), dim3(kSmallThreads), 0, stream, x, rows, K, \
                           ld, codes, scales, g, given);                                                        \
        break;
    switch (p) {
        NVFP4_QS(1)
        NVFP4_QS(2)
        NVFP4_QS(3)
        NVFP4_QS(4)
        NVFP4_QS(5)
        NVFP4_QS(6)
        NVFP4_QS(7)
        NVFP4_QS(8)
        default: return hipErrorInvalidValue;
    }
#undef NVFP4_QS
    return hipGetLastError();
}

int quantize_partials_count(int64_t rows, int64_t K) {
    const int64_t elems = rows * K;
    int64_t segs = (elems + kSegElems - 1) / kSegElems;
    if (segs < 1) segs = 1;
    return (int)(segs < kMaxPartials ? segs : kMaxPartials);
}

static int encode_grid(int64_t rows, int64_t K) {
    const int64_t nblk = rows * (K / 16);
    int64_t wg = (nblk + kQThreads - 1) / kQThreads;
    const int64_t cap = 256 * 16;  // ~16 workgroups per CU, the rest by grid stride
    if (wg > cap) wg = cap;
    return (int)(wg < 1 ? 1 : wg);
}

template <typename T>
static void launch_t(const T* xp, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales,
                     float* g, int given, float* partials, int n_partials, int vec, int vec_rows, int grid, int rht,
                     uint32_t signs, hipStream_t stream) {
    if (!rht) {
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<T>, dim3(n_partials), dim3(kQThreads), 0, stream,
                               xp, rows, cols, ld_x, partials, vec);
        hipLaunchKernelGGL((encode_t_kernel<T, kTEncode>), dim3(grid), dim3(kQThreads), 0, stream, xp, rows, cols,
                           ld_x, codes, scales, g, given, partials, n_partials, vec_rows, 0u, nullptr);
        return;
    }
    if (!given)
        hipLaunchKernelGGL((encode_t_kernel<T, kTAmaxRht>), dim3(n_partials), dim3(kQThreads), 0, stream, xp, rows,
                           cols, ld_x, nullptr, nullptr, nullptr, 0, nullptr, 0, vec_rows, signs, partials);
    hipLaunchKernelGGL((encode_t_kernel<T, kTEncodeRht>), dim3(grid), dim3(kQThreads), 0, stream, xp, rows, cols,
                       ld_x, codes, scales, g, given, partials, n_partials, vec_rows, signs, nullptr);
}

hipError_t launch_quantize_t(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t* codes, uint8_t* scales, float* g, int g_mode, float* partials, int n_partials,
                             hipStream_t stream, int rht, uint32_t signs) {
    const int given = (g_mode == NVFP4_G_GIVEN);
    if (rows == 0 || cols == 0) {
        if (!given) hipLaunchKernelGGL(write_unit_g_kernel, dim3(1), dim3(1), 0, stream, g);
        return hipGetLastError();
    }
    // 16-byte vector loads need an aligned base and (unless the tensor is dense) an aligned row stride
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ld_x == cols || (ld_x * esize) % 16 == 0);
    const int vec_rows = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ld_x * esize) % 16 == 0;
    const int64_t tcols = kTLanesC * (16 / esize);
    const int64_t tiles = ((rows + kTRows - 1) / kTRows) * ((cols + tcols - 1) / tcols);
    const int grid = (int)(tiles < (1 << 24) ? tiles : (1 << 24));   // one tile per workgroup in practice
    if (in_dtype == NVFP4_IN_BF16)
        launch_t(static_cast<const uint16_t*>(x), rows, cols, ld_x, codes, scales, g, given, partials, n_partials,
                 vec, vec_rows, grid, rht, signs, stream);
    else
        launch_t(static_cast<const float*>(x), rows, cols, ld_x, codes, scales, g, given, partials, n_partials,
                 vec, vec_rows, grid, rht, signs, stream);
    return hipGetLastError();
}

template <typename T>
static void launch_rows(const T* xp, int64_t rows, int64_t K, int64_t ld_x, uint8_t* codes, uint8_t* scales,
                        float* g, int given, float* partials, int n_partials, int grid, int rht, uint32_t signs,
                        hipStream_t stream) {
    if (!given) {
        if (rht)
            hipLaunchKernelGGL(amax_rht_kernel<T>, dim3(n_partials), dim3(kQThreads), 0, stream, xp, rows, K, ld_x,
                               signs, partials);
        else
            hipLaunchKernelGGL(amax_partials_kernel<T>, dim3(n_partials), dim3(kQThreads), 0, stream, xp, rows, K,
                               ld_x, partials, 1);
    }
    if (rht)
        hipLaunchKernelGGL((encode_kernel<T, true>), dim3(grid), dim3(kQThreads), 0, stream, xp, rows, K, ld_x, codes,
                           scales, g, given, partials, n_partials, signs);
    else
        hipLaunchKernelGGL((encode_kernel<T, false>), dim3(grid), dim3(kQThreads), 0, stream, xp, rows, K, ld_x,
                           codes, scales, g, given, partials, n_partials, 0u);
}

// ---------------------------------------------------------------------------
// Weight re-quantization for a training step: one weight W [n][k] read once,
// both packed operands written (the forward product's W along k, the backward
// dX = dY . W product's W^T along n), with one g.  The same lane patches as the
// x^T encoder (row blocks across neighbouring lanes, column blocks inside a
// lane), with the stores going straight to the packed blob order; the tiles
// also cover the padding rows of both blobs (zero input encodes to zero codes
// and zero scales), and the column scales and headers are written here too.
// ---------------------------------------------------------------------------
struct PackedOut {
    uint8_t *fwd, *bwd;                 // blob bases
    size_t f_codes, f_scales, f_cs;     // offsets inside the forward blob
    size_t b_codes, b_scales, b_cs;     // and the backward one
    int64_t ksf, ksb;                   // k-steps per row of each blob (k / 128, n / 128)
    int64_t n_pad, k_pad;               // padded row counts of the forward and backward blobs
};

__device__ __forceinline__ size_t code_unit(int64_t row, int64_t kb, int64_t ks_per_row) {
    return ((size_t)((row >> 4) * ks_per_row + (kb >> 3)) * 64 + (size_t)(((kb & 7) >> 1) * 16) + (size_t)(row & 15));
}
__device__ __forceinline__ size_t scale_unit(int64_t row, int64_t kb, int64_t ks_per_row) {
    return (size_t)((row >> 4) * ks_per_row + (kb >> 3)) * 16 + (size_t)(row & 15);
}

template <typename T>
__global__ __launch_bounds__(kQThreads) void pack_train_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                               int64_t ld, float* __restrict__ g_io, int g_given,
                                                               const float* __restrict__ partials, int n_partials,
                                                               int vec, PackedOut o) {
    __shared__ float s_senc, s_g;
    __shared__ float rtab[128];
    if (g_given) {
        if (threadIdx.x == 0) {
            s_g = g_io[0];
            s_senc = 1.0f / s_g;
        }
    } else {
        float pm = 0.0f;
        for (int i = threadIdx.x; i < n_partials; i += kQThreads) pm = fmaxf(pm, partials[i]);
        pm = block_max<kQThreads>(pm);
        if (threadIdx.x == 0) {
            const float g = global_scale_from_amax(pm);
            s_g = g;
            s_senc = 1.0f / g;
            if (blockIdx.x == 0) g_io[0] = g;
        }
    }
    __syncthreads();
    const float s_enc = s_senc, g = s_g;
    fill_recip_table(rtab, s_enc, threadIdx.x, kQThreads);
    __syncthreads();

    // column scales (g for real rows, 0 for padding) and the two headers
    for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < o.n_pad + o.k_pad;
         i += (int64_t)gridDim.x * kQThreads) {
        if (i < o.n_pad)
            reinterpret_cast<float*>(o.fwd + o.f_cs)[i] = i < rows ? g : 0.0f;
        else
            reinterpret_cast<float*>(o.bwd + o.b_cs)[i - o.n_pad] = i - o.n_pad < cols ? g : 0.0f;
    }
    if (blockIdx.x == 0 && threadIdx.x < 2) {
        uint8_t* blob = threadIdx.x == 0 ? o.fwd : o.bwd;
        uint32_t* h32 = reinterpret_cast<uint32_t*>(blob);
        int64_t* h64 = reinterpret_cast<int64_t*>(blob + 8);
        h32[0] = NVFP4_WEIGHT_MAGIC;
        h32[1] = NVFP4_WEIGHT_VERSION;
        h64[0] = threadIdx.x == 0 ? rows : cols;
        h64[1] = threadIdx.x == 0 ? cols : rows;
        h64[2] = threadIdx.x == 0 ? o.n_pad : o.k_pad;
        h64[3] = 1;
    }

    constexpr int kVec = 16 / (int)sizeof(T);
    constexpr int kRG = 64 / kTLanesC;
    constexpr int kTCols = kTLanesC * kVec;
    const int64_t tiles_r = (o.n_pad + kTRows - 1) / kTRows, tiles_c = (o.k_pad + kTCols - 1) / kTCols;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cl = lane % kTLanesC, rg = lane / kTLanesC;
    uint8_t* const fc = o.fwd + o.f_codes;
    uint8_t* const fs = o.fwd + o.f_scales;
    uint8_t* const bc = o.bwd + o.b_codes;
    uint8_t* const bs = o.bwd + o.b_scales;
    for (int64_t tile_id = blockIdx.x; tile_id < tiles_r * tiles_c; tile_id += gridDim.x) {
        const int64_t tr = tile_id % tiles_r, tc = tile_id / tiles_r;
        const int64_t r0 = tr * kTRows + (w * kRG + rg) * 16;
        const int64_t c0 = tc * kTCols + (int64_t)kVec * cl;
        if (r0 >= o.n_pad || c0 >= o.k_pad) continue;   // whole 16-row groups and 16-column blocks
        const T* src = x + r0 * ld + c0;
        T e[16][kVec];
        if (vec && r0 + 16 <= rows && c0 + kVec <= cols) {
#pragma unroll
            for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(e[i]) = *reinterpret_cast<const uint4*>(src + i * ld);
        } else {                           // padding, ragged edges or unaligned rows: element by element
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int k = 0; k < kVec; ++k)
                    e[i][k] = (r0 + i < rows && c0 + k < cols) ? src[i * ld + k] : T(0);
        }
        // row blocks (the forward operand, k = cols columns; its padding rows up to n_pad are written too):
        // 16/kVec neighbouring lanes share a block
        const int64_t kb = c0 >> 4;
        const int part = (int)((c0 >> (kVec == 8 ? 3 : 2)) & (16 / kVec - 1));   // which kVec-slice of the block
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (c0 >= cols) break;                  // (the lanes of a block agree: cols % 16 == 0)
            float v[kVec];
            float pm = 0.0f;
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                v[k] = elem_f32(e[i][k]);
                pm = fmaxf(pm, __builtin_fabsf(v[k]));
            }
            pm = fmaxf(pm, __shfl_xor(pm, 1, 64));
            if constexpr (kVec == 4) pm = fmaxf(pm, __shfl_xor(pm, 2, 64));
            uint32_t sc;
            const uint32_t wd = encode_part<kVec>(v, pm, s_enc, rtab, sc);
            const int64_t row = r0 + i;
            uint8_t* dst = fc + code_unit(row, kb, o.ksf) * 16 + (kb & 1) * 8 + part * (kVec / 2);
            if constexpr (kVec == 8)
                *reinterpret_cast<uint32_t*>(dst) = wd;
            else
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)wd;
            if (part == 0) fs[scale_unit(row, kb, o.ksf) * 8 + (kb & 7)] = (uint8_t)sc;
        }
        // column blocks (the backward operand, k = rows; its padding rows up to k_pad are written too):
        // output row c0 + k, block r0 / 16 along n
        const int64_t kbt = r0 >> 4;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            if (r0 >= rows) break;
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = elem_f32(e[i][k]);
            uint32_t lo, hi, sc;
            encode_block(v, block_amax(v), s_enc, rtab, lo, hi, sc);
            const int64_t c = c0 + k;
            *reinterpret_cast<uint2*>(bc + code_unit(c, kbt, o.ksb) * 16 + (kbt & 1) * 8) = make_uint2(lo, hi);
            bs[scale_unit(c, kbt, o.ksb) * 8 + (kbt & 7)] = (uint8_t)sc;
        }
    }
}

hipError_t launch_pack_train(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x, float* g,
                             int g_mode, float* partials, int n_partials, const nvfp4_weight_desc& df,
                             const nvfp4_weight_desc& db, hipStream_t stream) {
    const int given = (g_mode == NVFP4_G_GIVEN);
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ld_x * esize) % 16 == 0;
    const int vec_amax = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ld_x == cols || (ld_x * esize) % 16 == 0);
    PackedOut o;
    o.fwd = static_cast<uint8_t*>(const_cast<void*>(df.blob));   // the blobs being written
    o.bwd = static_cast<uint8_t*>(const_cast<void*>(db.blob));
    o.f_codes = df.codes_offset; o.f_scales = df.scales_offset; o.f_cs = df.colscale_offset;
    o.b_codes = db.codes_offset; o.b_scales = db.scales_offset; o.b_cs = db.colscale_offset;
    o.ksf = df.k / kPackK;
    o.ksb = db.k / kPackK;
    o.n_pad = df.n_padded;
    o.k_pad = db.n_padded;
    const int64_t tcols = kTLanesC * (16 / esize);
    const int64_t tiles = ((o.n_pad + kTRows - 1) / kTRows) * ((o.k_pad + tcols - 1) / tcols);
    const int grid = (int)(tiles < (1 << 24) ? tiles : (1 << 24));
    if (in_dtype == NVFP4_IN_BF16) {
        const uint16_t* xp = static_cast<const uint16_t*>(x);
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<uint16_t>, dim3(n_partials), dim3(kQThreads), 0, stream, xp,
                               rows, cols, ld_x, partials, vec_amax);
        hipLaunchKernelGGL(pack_train_kernel<uint16_t>, dim3(grid), dim3(kQThreads), 0, stream, xp, rows, cols, ld_x,
                           g, given, partials, n_partials, vec, o);
    } else {
        const float* xp = static_cast<const float*>(x);
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<float>, dim3(n_partials), dim3(kQThreads), 0, stream, xp, rows,
                               cols, ld_x, partials, vec_amax);
        hipLaunchKernelGGL(pack_train_kernel<float>, dim3(grid), dim3(kQThreads), 0, stream, xp, rows, cols, ld_x, g,
                           given, partials, n_partials, vec, o);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_both(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, float* g,
                                int g_mode, float* partials, int n_partials, hipStream_t stream) {
    const int given = (g_mode == NVFP4_G_GIVEN);
    if (rows == 0 || cols == 0) {
        if (!given) hipLaunchKernelGGL(write_unit_g_kernel, dim3(1), dim3(1), 0, stream, g);
        return hipGetLastError();
    }
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ld_x == cols || (ld_x * esize) % 16 == 0);
    const int vec_rows = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ld_x * esize) % 16 == 0;
    const int64_t tcols = kTLanesC * (16 / esize);
    const int64_t tiles = ((rows + kTRows - 1) / kTRows) * ((cols + tcols - 1) / tcols);
    const int grid = (int)(tiles < (1 << 24) ? tiles : (1 << 24));
    if (in_dtype == NVFP4_IN_BF16) {
        const uint16_t* xp = static_cast<const uint16_t*>(x);
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<uint16_t>, dim3(n_partials), dim3(kQThreads), 0, stream, xp,
                               rows, cols, ld_x, partials, vec);
        hipLaunchKernelGGL((encode_t_kernel<uint16_t, kTBoth>), dim3(grid), dim3(kQThreads), 0, stream, xp, rows,
                           cols, ld_x, codes_t, scales_t, g, given, partials, n_partials, vec_rows, 0u, nullptr,
                           codes, scales);
    } else {
        const float* xp = static_cast<const float*>(x);
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<float>, dim3(n_partials), dim3(kQThreads), 0, stream, xp, rows,
                               cols, ld_x, partials, vec);
        hipLaunchKernelGGL((encode_t_kernel<float, kTBoth>), dim3(grid), dim3(kQThreads), 0, stream, xp, rows, cols,
                           ld_x, codes_t, scales_t, g, given, partials, n_partials, vec_rows, 0u, nullptr, codes,
                           scales);
    }
    return hipGetLastError();
}

hipError_t launch_kv_fp8(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                         float* scale, int s_mode, float* partials, int n_partials, hipStream_t stream) {
    const int given = (s_mode == NVFP4_G_GIVEN);
    if (rows == 0 || cols == 0) {
        if (!given) hipLaunchKernelGGL(write_unit_g_kernel, dim3(1), dim3(1), 0, stream, scale);
        return hipGetLastError();
    }
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const bool x16 = reinterpret_cast<uintptr_t>(x) % 16 == 0;
    // vector runs: 16-byte aligned input rows (or a dense tensor) and 8-byte aligned output runs
    const int vec_in = x16 && (ld_x == cols || (ld_x * esize) % 16 == 0);
    const int vec = vec_in && (reinterpret_cast<uintptr_t>(codes) % 8 == 0) && cols % 8 == 0 &&
                    (ld_x * esize) % 16 == 0;
    const int64_t runs = rows * ((cols + 7) / 8);
    int64_t wg = (runs + kQThreads - 1) / kQThreads;
    if (wg > 256 * 16) wg = 256 * 16;
    if (in_dtype == NVFP4_IN_BF16) {
        const uint16_t* xp = static_cast<const uint16_t*>(x);
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<uint16_t>, dim3(n_partials), dim3(kQThreads), 0, stream, xp,
                               rows, cols, ld_x, partials, vec_in);
        hipLaunchKernelGGL(kv_fp8_kernel<uint16_t>, dim3((int)wg), dim3(kQThreads), 0, stream, xp, rows, cols, ld_x,
                           codes, scale, given, partials, n_partials, vec);
    } else {
        const float* xp = static_cast<const float*>(x);
        if (!given)
            hipLaunchKernelGGL(amax_partials_kernel<float>, dim3(n_partials), dim3(kQThreads), 0, stream, xp, rows,
                               cols, ld_x, partials, vec_in);
        hipLaunchKernelGGL(kv_fp8_kernel<float>, dim3((int)wg), dim3(kQThreads), 0, stream, xp, rows, cols, ld_x,
                           codes, scale, given, partials, n_partials, vec);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x,
                           uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                           float* partials, int n_partials, hipStream_t stream, int rht, uint32_t signs) {
    const int given = (g_mode == NVFP4_G_GIVEN);
    if (rows == 0) {
        if (!given) hipLaunchKernelGGL(write_unit_g_kernel, dim3(1), dim3(1), 0, stream, g);
        return hipGetLastError();
    }
    const int p = rht ? 0 : small_blocks_per_thread(rows, K, ld_x, in_dtype);   // the one-launch path has no RHT
    if (p > 0) {
        if (in_dtype == NVFP4_IN_BF16)
            return launch_small<uint16_t>(p, static_cast<const uint16_t*>(x), rows, K, ld_x, codes, scales, g, given,
                                          stream);
        if (p <= 4)
            return launch_small<float>(p, static_cast<const float*>(x), rows, K, ld_x, codes, scales, g, given,
                                       stream);
    }
    const int grid = encode_grid(rows, K);
    if (in_dtype == NVFP4_IN_BF16)
        launch_rows(static_cast<const uint16_t*>(x), rows, K, ld_x, codes, scales, g, given, partials, n_partials,
                    grid, rht, signs, stream);
    else
        launch_rows(static_cast<const float*>(x), rows, K, ld_x, codes, scales, g, given, partials, n_partials,
                    grid, rht, signs, stream);
    return hipGetLastError();
}

}  // namespace nvfp4
