// NVFP4 activation/weight quantizer for gfx950.
//
// The per-tensor scale is a global dependency of every block's encoding, so a
// large tensor takes two kernels:
//   1. amax: each workgroup reduces max|x| over its share of the tensor and
//      writes one partial (no atomics, no initialised memory needed).
//   2. encode: every workgroup reduces the partials itself (a few KB from L2),
//      derives g and s_enc = fl32(1/g), and encodes 16-element blocks along K:
//      bamax -> E4M3 scale of fl32(fl32(bamax*s_enc)/6) -> r = fl32(s_enc/S)
//      (from a 128-entry table per workgroup)
//      -> E2M1 code of fl32(x*r) per element -> two codes per byte.
// A small tensor takes one kernel whose workgroups each reduce the whole tensor
// (quantize_small_kernel); one of up to 64 MB takes one kernel whose workgroups
// keep their shares in registers while they exchange their maxima
// (quantize_resident_kernel), so it is read once.
// The block structure and per-tensor scale follow "Why Gated DeltaNet Survives
// 4-Bit Quantization" (sections "Why the 'Fragile' Recurrence is Actually
// Robust" and "Critical Lessons for Model Serving").  Every decision is taken
// in IEEE FP32 with one rounding per operation (contraction disabled below),
// so codes and scales are bit-for-bit reproducible.
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "launch_tag.h"

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
    // each workgroup streams one contiguous run of segments (measured on MI355X over 1 GiB: 6.9 TB/s with
    // streaming loads, against 5.0-5.6 TB/s for segments dealt out round-robin over the workgroups)
    const int64_t per = (nseg + gridDim.x - 1) / gridDim.x;
    const int64_t s_end = min(nseg, ((int64_t)blockIdx.x + 1) * per);
    float m = 0.0f;
    for (int64_t s = (int64_t)blockIdx.x * per; s < s_end; ++s) {
        const int64_t r = s / seg_per_row;
        const int64_t c0 = (s - r * seg_per_row) * kSegElems;
        const T* row = x + r * ld;
#pragma unroll
        for (int u = 0; u < kSegVec; ++u) {
            const int64_t c = c0 + ((int64_t)u * kQThreads + threadIdx.x) * 8;
            if (vec && c + 8 <= K) {
                float v[8];
                load8_stream(row + c, v);
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

// Per-workgroup max |x| of a dense tensor whose base is 16-byte aligned, read
// as n16 16-byte vectors: each workgroup streams one contiguous chunk of whole
// steps (kAmaxVec vectors per thread in flight, streaming loads) and reduces
// the magnitudes' bit patterns, which order like the values for finite inputs
// (two bf16 magnitudes per packed 16-bit max).  Measured on MI355X: 6.9 TB/s
// for this read pattern over 1 GiB.
constexpr int kAmaxVec = 8;
template <typename T>
__global__ __launch_bounds__(kQThreads) void amax_dense_kernel(const uint4* __restrict__ x, int64_t n16,
                                                               float* __restrict__ partials) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    constexpr int64_t kStep = (int64_t)kQThreads * kAmaxVec;
    const int64_t per = (n16 + (int64_t)gridDim.x * kStep - 1) / ((int64_t)gridDim.x * kStep) * kStep;
    const int64_t end = min(n16, ((int64_t)blockIdx.x + 1) * per);
    u16x2 m2 = {0, 0};
    uint32_t m = 0;
    for (int64_t i0 = (int64_t)blockIdx.x * per + threadIdx.x; i0 < end; i0 += kStep) {
        uint4 v[kAmaxVec];
#pragma unroll
        for (int u = 0; u < kAmaxVec; ++u) {
            const int64_t i = i0 + (int64_t)u * kQThreads;
            v[u] = i < end ? load16_stream(x + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kAmaxVec; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (sizeof(T) == 2)
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
                else
                    m = max(m, w[j] & 0x7FFFFFFFu);
            }
        }
    }
    if constexpr (sizeof(T) == 2) m = (uint32_t)max(m2.x, m2.y) << 16;
    const float r = block_max<kQThreads>(__uint_as_float(m));
    if (threadIdx.x == 0) partials[blockIdx.x] = r;
}

// Per-workgroup max |v| over transformed blocks (the global amax of the
// transformed tensor), one partial per workgroup, over one contiguous run of blocks.
template <typename T>
__global__ __launch_bounds__(kQThreads) void amax_rht_kernel(const T* __restrict__ x, int64_t rows, int64_t K,
                                                             int64_t ld, uint32_t signs, float* __restrict__ partials) {
    const int64_t bpr = K / 16, nblk = rows * bpr;
    const int64_t per = (nblk + (int64_t)gridDim.x * kQThreads - 1) / ((int64_t)gridDim.x * kQThreads) * kQThreads;
    const int64_t b_end = min(nblk, ((int64_t)blockIdx.x + 1) * per);
    float m = 0.0f;
    for (int64_t b = (int64_t)blockIdx.x * per + threadIdx.x; b < b_end; b += kQThreads) {
        const int64_t r = b / bpr;
        const T* src = x + r * ld + (b - r * bpr) * 16;
        float v[16];
        load8_stream(src, v);
        load8_stream(src + 8, v + 8);
        rht16(v, signs);
        m = fmaxf(m, block_amax(v));
    }
    m = block_max<kQThreads>(m);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Block b's 8 code bytes and its scale byte.
__device__ __forceinline__ void store_code_block(uint8_t* codes, uint8_t* scales, int64_t b, uint32_t lo, uint32_t hi,
                                                 uint32_t S) {
    *reinterpret_cast<uint2*>(codes + b * 8) = make_uint2(lo, hi);
    scales[b] = (uint8_t)S;
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
    auto src_of = [&](int64_t b) -> const T* {
        if (dense) return x + b * 16;
        const int64_t r = b / bpr;
        return x + r * ld + (b - r * bpr) * 16;
    };
    // One contiguous run of blocks per workgroup (whole steps of 2 * kQThreads blocks), two blocks per
    // thread in flight.  Plain loads and stores: on MI355X (32768 x 16384 bf16, g given) this takes
    // 273 us, the same as blocks dealt out round-robin, and 284-308 us with streaming loads or stores,
    // which help only the read-only amax pass.
    constexpr int64_t kStep = 2 * kQThreads;
    const int64_t per = (nblk + (int64_t)gridDim.x * kStep - 1) / ((int64_t)gridDim.x * kStep) * kStep;
    const int64_t b_end = min(nblk, ((int64_t)blockIdx.x + 1) * per);
    for (int64_t b0 = (int64_t)blockIdx.x * per + threadIdx.x; b0 < b_end; b0 += kStep) {
        const int64_t b1 = b0 + kQThreads;
        const bool two = b1 < b_end;
        float v0[16], v1[16];
        load8(src_of(b0), v0);
        load8(src_of(b0) + 8, v0 + 8);
        if (two) {
            load8(src_of(b1), v1);
            load8(src_of(b1) + 8, v1 + 8);
        }
        uint32_t lo, hi, S;
        if (RHT) rht16(v0, signs);
        encode_block(v0, block_amax(v0), s_enc, rtab, lo, hi, S);
        store_code_block(codes, scales, b0, lo, hi, S);
        if (two) {
            if (RHT) rht16(v1, signs);
            encode_block(v1, block_amax(v1), s_enc, rtab, lo, hi, S);
            store_code_block(codes, scales, b1, lo, hi, S);
        }
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

// One lane's patch e (rows r0 .. r0+15, columns c0 .. c0+kVec-1 of x) through
// the transposed encoder: in kTBoth the row blocks first (a 16-column row block
// spans 16/kVec neighbouring lanes, which combine their maxima by lane exchange
// and each encode their own kVec elements), then each column's block of x^T
// (transformed first in the RHT modes); kTAmaxRht only raises m.
template <typename T, int MODE, int kVec>
__device__ __forceinline__ void encode_t_patch(const T (&e)[16][kVec], int64_t r0, int64_t c0, int64_t rows,
                                               int64_t cols, float s_enc, const float* rtab, uint32_t signs,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                               uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
                                               float& m) {
    if constexpr (MODE == kTBoth) {
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
        encode_t_patch<T, MODE, kVec>(e, r0, c0, rows, cols, s_enc, rtab, signs, codes, scales, codes_r, scales_r, m);
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

// ---------------------------------------------------------------------------
// One pass for a tensor that fits the register files (up to 64 MB): every
// workgroup (one per compute unit, all resident at once) loads its share of
// the blocks into registers, reduces its max|x| and publishes it; every
// workgroup then reads all the published maxima, derives the same g and
// encodes its blocks from its registers, so x is read from memory once
// instead of twice.  The exchange spans all XCDs, so both words of a record
// are device-scope atomics (stored through to memory, loaded from it): the
// writer stores the max, waits for that store to complete, then stores the
// launch tag; a reader that has loaded the current tag loads the max after
// that load completed.  Only these atomic words cross workgroups, so no L2
// write-back or invalidate is needed (with them the exchange took ~5 us
// longer).  A workgroup whose wait exceeds a bound (a workgroup not resident,
// if another kernel holds compute units) reduces max|x| over the whole tensor
// itself: the same g.
// ---------------------------------------------------------------------------
struct AmaxRecord {
    uint32_t max_bits;
    uint32_t pad;
    uint64_t tag;
};
constexpr int kResThreads = 1024;
// records of one launch fit the partials' part of the workspace (256 of them)
constexpr int kResMaxGrid = kMaxAmaxPartials * (int)sizeof(float) / (int)sizeof(AmaxRecord);
template <typename T>
struct ResBlocks : std::integral_constant<int, sizeof(T) == 2 ? 8 : 4> {};   // 64 raw registers per thread
constexpr int kResDefaultPolls = 1 << 15;

// The one-pass kernels' exchange: this workgroup's max|x| m (the same in every
// thread) is published, and the tensor's max|x| returned (the same value in
// every workgroup), from the records of all the grid's workgroups, or, if they
// do not all arrive within `polls`, from the whole tensor x [rows][K] (row
// stride ld) read by this workgroup.  *s_fail: a shared word, 0 on entry.
template <typename T, bool RHT = false>
__device__ float exchange_amax(float m, AmaxRecord* rec, int polls, const T* __restrict__ x, int64_t rows, int64_t K,
                               int64_t ld, int* s_fail, uint32_t signs = 0) {
    const int G = (int)gridDim.x;
    const uint64_t tag = launch_tag();
    if (threadIdx.x == 0) {
        __hip_atomic_store(&rec[blockIdx.x].max_bits, __float_as_uint(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __hip_atomic_store(&rec[blockIdx.x].tag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // thread t waits for record t, then (after the barrier, so every record is in) loads its max
    if ((int)threadIdx.x < G) {
        bool ok = false;
        for (int i = 0; i < polls && !ok; ++i) {
            ok = __hip_atomic_load(&rec[threadIdx.x].tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
            if (!ok) __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) *s_fail = 1;
    }
    __syncthreads();
    const float mt = (int)threadIdx.x < G && !*s_fail
                         ? __uint_as_float(__hip_atomic_load(&rec[threadIdx.x].max_bits, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT))
                         : 0.0f;
    float amax = block_max<kResThreads>(mt);
    if (*s_fail) {   // (uniform: written before the barriers of block_max)
        float w = 0.0f;
        if constexpr (RHT) {   // max |v| over the transformed blocks, one block per thread at a time
            const int64_t bpr = K / 16, nblk = rows * bpr;
            for (int64_t b = threadIdx.x; b < nblk; b += kResThreads) {
                const int64_t r = b / bpr;
                const T* src = x + r * ld + (b - r * bpr) * 16;
                float v[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = elem_f32(src[i]);
                rht16(v, signs);
                w = fmaxf(w, block_amax(v));
            }
        } else {
            for (int64_t r = threadIdx.x / (kResThreads / 64); r < rows; r += 64)   // 64 rows at a time,
                for (int64_t c = threadIdx.x % (kResThreads / 64); c < K; c += kResThreads / 64)   // 16 lanes a row
                    w = fmaxf(w, __builtin_fabsf(elem_f32(x[r * ld + c])));
        }
        amax = block_max<kResThreads>(w);
    }
    return amax;
}

template <typename T, bool RHT>
__global__ __launch_bounds__(kResThreads) void quantize_resident_kernel(const T* __restrict__ x, int64_t rows,
                                                                        int64_t K, int64_t ld,
                                                                        uint8_t* __restrict__ codes,
                                                                        uint8_t* __restrict__ scales,
                                                                        float* __restrict__ g_out, AmaxRecord* rec,
                                                                        int polls, uint32_t signs) {
    constexpr int R = ResBlocks<T>::value;
    __shared__ int s_fail;
    __shared__ float rtab[128];
    if (threadIdx.x == 0) s_fail = 0;   // (ordered before its uses by the barriers in block_max)
    const int G = (int)gridDim.x;
    const uint32_t bpr = (uint32_t)(K / 16), nblk = (uint32_t)rows * bpr;
    const uint32_t per = (nblk + (uint32_t)G - 1) / (uint32_t)G;
    const uint32_t b0 = blockIdx.x * per, b1 = min(nblk, b0 + per);
    const rsrc_t rx = make_rsrc(x, (uint64_t)rows * ld * sizeof(T));
    const bool dense = (ld == K);
    RawBlock<T> raw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {   // branch-free: blocks past the share read as zero
        const uint32_t b = b0 + threadIdx.x + (uint32_t)i * kResThreads;
        uint32_t off = kOutOfBounds;
        if (b < b1) {
            const uint32_t r = dense ? 0u : b / bpr, kb = dense ? b : b - r * bpr;
            off = (uint32_t)(((int64_t)r * ld + (int64_t)kb * 16) * (int64_t)sizeof(T));
        }
#pragma unroll
        for (int q = 0; q < (int)(sizeof(RawBlock<T>) / 16); ++q)
            raw[i].v[q] = bload16(rx, off, (uint32_t)q * 16);
    }
    // block maxima from the raw bits (finite magnitudes order like their bit patterns), without widening;
    // with the transform, of each block widened and transformed (the packed block stays, and is
    // transformed again for the encoding)
    float bm[R], m = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if constexpr (RHT) {
            float v[16];
            widen(raw[i], v);
            rht16(v, signs);
            bm[i] = block_amax(v);
            m = fmaxf(m, bm[i]);
            continue;
        }
        uint32_t mb = 0;
#pragma unroll
        for (int q = 0; q < (int)(sizeof(RawBlock<T>) / 16); ++q) {
            const uint32_t w[4] = {raw[i].v[q].x, raw[i].v[q].y, raw[i].v[q].z, raw[i].v[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (sizeof(T) == 2) {
                    mb = max(mb, (w[e] & 0x7FFFu) << 16);
                    mb = max(mb, w[e] & 0x7FFF0000u);
                } else {
                    mb = max(mb, w[e] & 0x7FFFFFFFu);
                }
            }
        }
        bm[i] = __uint_as_float(mb);
        m = fmaxf(m, bm[i]);
    }
    m = block_max<kResThreads>(m);
    const float amax = exchange_amax<T, RHT>(m, rec, polls, x, rows, K, ld, &s_fail, signs);
    const float g = global_scale_from_amax(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) g_out[0] = g;
    const float s_enc = 1.0f / g;
    fill_recip_table(rtab, s_enc, threadIdx.x, kResThreads);
    __syncthreads();
    // (the raw blocks stay packed until here: widened all at once they would not fit the registers)
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int q = 0; q < (int)(sizeof(RawBlock<T>) / 16); ++q)
            asm volatile("" : "+v"(raw[i].v[q].x), "+v"(raw[i].v[q].y), "+v"(raw[i].v[q].z), "+v"(raw[i].v[q].w));
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t b = b0 + threadIdx.x + (uint32_t)i * kResThreads;
        if (b < b1) {
            float v[16];
            widen(raw[i], v);
            if constexpr (RHT) rht16(v, signs);
            uint32_t lo, hi, S;
            encode_block(v, bm[i], s_enc, rtab, lo, hi, S);
            store_code_block(codes, scales, (int64_t)b, lo, hi, S);
        }
    }
}

// The one-pass form of the transposed encoder (and of the encoding both ways):
// each of the first nq (1, 2 or 4) 256-thread quarters of a workgroup holds one
// tile of the transposed encoder (512 rows x 8 lanes' columns, one 16-row patch
// per lane) in registers, quarters stacked along the rows and workgroups
// numbered column-major as there (the host takes the smallest nq whose grid
// fits one workgroup per compute unit, so the encoding after the exchange is
// spread over as many units as it can be); the workgroups exchange their maxima
// as in quantize_resident_kernel, then every lane encodes its patch from
// registers. Quarters past nq, and lanes whose 16 rows or kVec columns lie past
// the tensor, load nothing, publish 0 and encode nothing.
template <typename T, int MODE>
__global__ __launch_bounds__(kResThreads) void quantize_t_resident_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ g_out, AmaxRecord* rec, int polls,
    uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r, int nq) {
    constexpr int kVec = 16 / (int)sizeof(T);
    constexpr int kRG = 64 / kTLanesC;
    constexpr int kTCols = kTLanesC * kVec;
    __shared__ int s_fail;
    __shared__ float rtab[128];
    if (threadIdx.x == 0) s_fail = 0;   // (ordered before its uses by the barriers in block_max)
    const int64_t tiles_r = (rows + (int64_t)nq * kTRows - 1) / ((int64_t)nq * kTRows);
    const int64_t tr = blockIdx.x % tiles_r, tc = blockIdx.x / tiles_r;
    const int q = threadIdx.x / kQThreads, t = threadIdx.x % kQThreads;
    const int lane = t & 63, w = t >> 6;
    const int cl = lane % kTLanesC, rg = lane / kTLanesC;
    const int64_t r0 = (tr * nq + q) * kTRows + (w * kRG + rg) * 16;   // this lane's 16 rows
    const int64_t c0 = tc * kTCols + (int64_t)kVec * cl;                // and kVec columns
    const bool live = q < nq && r0 < rows && c0 < cols;
    // the patch, row i's kVec elements packed in pu[i] (cols is a multiple of kVec here; a lane past the
    // tensor reads zeros through the buffer bounds)
    const rsrc_t rx = make_rsrc(x, (uint64_t)rows * ld * sizeof(T));
    const uint32_t off = live ? (uint32_t)((r0 * ld + c0) * (int64_t)sizeof(T)) : kOutOfBounds;
    uint4 pu[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pu[i] = bload16(rx, live ? off + (uint32_t)(i * ld * (int64_t)sizeof(T)) : kOutOfBounds, 0);
    // max |x| of the patch from the bits (finite magnitudes order like their bit patterns)
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint4 u = pu[i];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(T) == 2) {
                mb = max(mb, (wd[j] & 0x7FFFu) << 16);
                mb = max(mb, wd[j] & 0x7FFF0000u);
            } else {
                mb = max(mb, wd[j] & 0x7FFFFFFFu);
            }
        }
    }
    const float m = block_max<kResThreads>(__uint_as_float(mb));
    const float amax = exchange_amax<T>(m, rec, polls, x, rows, cols, ld, &s_fail);
    const float g = global_scale_from_amax(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) g_out[0] = g;
    const float s_enc = 1.0f / g;
    fill_recip_table(rtab, s_enc, threadIdx.x, kResThreads);
    __syncthreads();
    // (the patch stays packed until here)
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(pu[i].x), "+v"(pu[i].y), "+v"(pu[i].z), "+v"(pu[i].w));
    float unused = 0.0f;
    if (live)
        encode_t_patch<T, MODE, kVec>(*reinterpret_cast<const T(*)[16][kVec]>(pu), r0, c0, rows, cols, s_enc, rtab,
                                      0u, codes, scales, codes_r, scales_r, unused);
}

// Poll bound of the one-pass kernels' exchange (NVFP4_AMAX_POLLS overrides it: 0 forces the local path,
// for tests).
static int resident_polls() {
    int polls = kResDefaultPolls;
    if (const char* e = std::getenv("NVFP4_AMAX_POLLS")) polls = std::atoi(e);
    return polls;
}

// Compute units of the current device (cached per device).
static int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of the one-pass transposed encoder for this tensor, or 0 when it does not apply.
static int resident_t_grid(int64_t rows, int64_t cols, int64_t ld, int in_dtype, const void* x, const float* partials,
                           int n_partials, int* nq) {
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (n_partials < kMaxAmaxPartials || reinterpret_cast<uintptr_t>(partials) % 16 != 0) return 0;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || (ld * esize) % 16 != 0 || (cols * esize) % 16 != 0) return 0;
    if (rows * ld * esize > INT32_MAX) return 0;
    const int cus = cu_count();
    const int64_t cap = cus < kResMaxGrid ? cus : kResMaxGrid;
    const int64_t tcols = kTLanesC * (16 / esize), tiles_c = (cols + tcols - 1) / tcols;
    // the fewest quarters per workgroup whose grid still fits one workgroup per compute unit
    for (int q = 1; q <= kResThreads / kQThreads; q *= 2) {
        const int64_t tiles = (rows + (int64_t)q * kTRows - 1) / ((int64_t)q * kTRows) * tiles_c;
        if (tiles <= cap) {
            *nq = q;
            return (int)tiles;
        }
    }
    return 0;
}

// Workgroups of the one-pass training-weight packer over the padded sizes
// n_pad x k_pad, or 0 when it does not apply (x aligned for 16-byte loads).
static int resident_pack_grid(int64_t n_pad, int64_t k_pad, int64_t rows, int64_t ld, int esize, int vec,
                              const float* partials, int n_partials, int* nq) {
    if (!vec || n_partials < kMaxAmaxPartials || reinterpret_cast<uintptr_t>(partials) % 16 != 0) return 0;
    if (rows * ld * esize > INT32_MAX) return 0;
    const int cus = cu_count();
    const int64_t cap = cus < kResMaxGrid ? cus : kResMaxGrid;
    const int64_t tcols = kTLanesC * (16 / esize), tiles_c = (k_pad + tcols - 1) / tcols;
    for (int q = 1; q <= kResThreads / kQThreads; q *= 2) {   // the fewest quarters whose grid fits
        const int64_t tiles = (n_pad + (int64_t)q * kTRows - 1) / ((int64_t)q * kTRows) * tiles_c;
        if (tiles <= cap) {
            *nq = q;
            return (int)tiles;
        }
    }
    return 0;
}

// Workgroups of the one-pass path for this tensor, or 0 when it does not apply.
static int resident_grid(int64_t rows, int64_t K, int64_t ld, int in_dtype, const void* x, const float* partials,
                         int n_partials) {
    const int esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    const int per_thread = in_dtype == NVFP4_IN_BF16 ? ResBlocks<uint16_t>::value : ResBlocks<float>::value;
    // the records need the whole partials area, aligned for their 64-bit tags
    if (n_partials < kMaxAmaxPartials || reinterpret_cast<uintptr_t>(partials) % 16 != 0) return 0;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || (ld * esize) % 16 != 0) return 0;
    if (rows * ld * esize > INT32_MAX) return 0;
    const int cus = cu_count();
    const int grid = cus < kResMaxGrid ? cus : kResMaxGrid;
    if (grid < 1) return 0;
    const int64_t nblk = rows * (K / 16);
    return nblk <= (int64_t)grid * kResThreads * per_thread ? grid : 0;
}

int quantize_partials_count(int64_t rows, int64_t K) {
    const int64_t elems = rows * K;
    int64_t segs = (elems + kSegElems - 1) / kSegElems;
    if (segs < 1) segs = 1;
    return (int)(segs < kMaxPartials ? segs : kMaxPartials);
}

static int encode_grid(int64_t rows, int64_t K) {
    const int64_t nblk = rows * (K / 16);
    int64_t wg = (nblk + 2 * kQThreads - 1) / (2 * kQThreads);   // two blocks per thread at least
    const int64_t cap = 256 * 16;  // ~16 workgroups per CU, each a longer contiguous run beyond that
    if (wg > cap) wg = cap;
    return (int)(wg < 1 ? 1 : wg);
}

template <typename T>
static void launch_t(const T* xp, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales,
                     float* g, int given, float* partials, int n_partials, int vec, int vec_rows, int grid, int rht,
                     uint32_t signs, hipStream_t stream) {
    if (!rht) {
        int nq = 0;
        const int rg = given ? 0 : resident_t_grid(rows, cols, ld_x, sizeof(T) == 2 ? NVFP4_IN_BF16 : NVFP4_IN_F32,
                                                   xp, partials, n_partials, &nq);
        if (rg > 0) {
            hipLaunchKernelGGL((quantize_t_resident_kernel<T, kTEncode>), dim3(rg), dim3(kResThreads), 0, stream, xp,
                               rows, cols, ld_x, codes, scales, g, reinterpret_cast<AmaxRecord*>(partials),
                               resident_polls(), nullptr, nullptr, nq);
            return;
        }
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
        else if (ld_x == K && reinterpret_cast<uintptr_t>(xp) % 16 == 0)
            hipLaunchKernelGGL(amax_dense_kernel<T>, dim3(n_partials), dim3(kQThreads), 0, stream,
                               reinterpret_cast<const uint4*>(xp), rows * K * (int64_t)sizeof(T) / 16, partials);
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

// One lane's 16-row x kVec-column patch e (rows r0.., columns c0..; zero past
// x, up to the padded sizes) into both packed blobs: its row-block parts (the
// 16/kVec neighbouring lanes of a block combine their maxima) and its kVec
// column blocks.
template <typename T, int kVec>
__device__ __forceinline__ void pack_train_patch(const T (&e)[16][kVec], int64_t r0, int64_t c0, int64_t rows,
                                                 int64_t cols, float s_enc, const float* rtab, const PackedOut& o) {
    uint8_t* const fc = o.fwd + o.f_codes;
    uint8_t* const fs = o.fwd + o.f_scales;
    uint8_t* const bc = o.bwd + o.b_codes;
    uint8_t* const bs = o.bwd + o.b_scales;
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

// Both blobs' column scales (g for real rows, 0 for padding) and headers, by
// thread `tid` of `nthreads`.
__device__ __forceinline__ void pack_train_headers(const PackedOut& o, int64_t rows, int64_t cols, float g,
                                                   int64_t tid, int64_t nthreads) {
    for (int64_t i = tid; i < o.n_pad + o.k_pad; i += nthreads) {
        if (i < o.n_pad)
            reinterpret_cast<float*>(o.fwd + o.f_cs)[i] = i < rows ? g : 0.0f;
        else
            reinterpret_cast<float*>(o.bwd + o.b_cs)[i - o.n_pad] = i - o.n_pad < cols ? g : 0.0f;
    }
    if (tid < 2) {
        uint8_t* blob = tid == 0 ? o.fwd : o.bwd;
        uint32_t* h32 = reinterpret_cast<uint32_t*>(blob);
        int64_t* h64 = reinterpret_cast<int64_t*>(blob + 8);
        h32[0] = NVFP4_WEIGHT_MAGIC;
        h32[1] = NVFP4_WEIGHT_VERSION;
        h64[0] = tid == 0 ? rows : cols;
        h64[1] = tid == 0 ? cols : rows;
        h64[2] = tid == 0 ? o.n_pad : o.k_pad;
        h64[3] = 1;
    }
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

    pack_train_headers(o, rows, cols, g, (int64_t)blockIdx.x * kQThreads + threadIdx.x, (int64_t)gridDim.x * kQThreads);

    constexpr int kVec = 16 / (int)sizeof(T);
    constexpr int kRG = 64 / kTLanesC;
    constexpr int kTCols = kTLanesC * kVec;
    const int64_t tiles_r = (o.n_pad + kTRows - 1) / kTRows, tiles_c = (o.k_pad + kTCols - 1) / kTCols;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cl = lane % kTLanesC, rg = lane / kTLanesC;
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
        pack_train_patch<T, kVec>(e, r0, c0, rows, cols, s_enc, rtab, o);
    }
}

// The one-pass form of the training-weight packer (g computed): each of the
// first nq quarters of a 1024-thread workgroup holds one tile of patches of
// pack_train_kernel in registers (quarters stacked along the rows, workgroups
// numbered column-major, over the padded sizes), the workgroups exchange their
// maxima as in quantize_resident_kernel, then every lane writes its patch into
// both blobs from registers.  Patches lie wholly inside W or wholly in the
// padding (n and k are multiples of 128); padding patches load zeros.
template <typename T>
__global__ __launch_bounds__(kResThreads) void pack_train_resident_kernel(const T* __restrict__ x, int64_t rows,
                                                                          int64_t cols, int64_t ld,
                                                                          float* __restrict__ g_out, AmaxRecord* rec,
                                                                          int polls, PackedOut o, int nq) {
    constexpr int kVec = 16 / (int)sizeof(T);
    constexpr int kRG = 64 / kTLanesC;
    constexpr int kTCols = kTLanesC * kVec;
    __shared__ int s_fail;
    __shared__ float rtab[128];
    if (threadIdx.x == 0) s_fail = 0;   // (ordered before its uses by the barriers in block_max)
    const int64_t tiles_r = (o.n_pad + (int64_t)nq * kTRows - 1) / ((int64_t)nq * kTRows);
    const int64_t tr = blockIdx.x % tiles_r, tc = blockIdx.x / tiles_r;
    const int q = threadIdx.x / kQThreads, t = threadIdx.x % kQThreads;
    const int lane = t & 63, w = t >> 6;
    const int cl = lane % kTLanesC, rg = lane / kTLanesC;
    const int64_t r0 = (tr * nq + q) * kTRows + (w * kRG + rg) * 16;
    const int64_t c0 = tc * kTCols + (int64_t)kVec * cl;
    const bool live = q < nq && r0 < o.n_pad && c0 < o.k_pad;
    const bool in_x = live && r0 < rows && c0 < cols;
    const rsrc_t rx = make_rsrc(x, (uint64_t)rows * ld * sizeof(T));
    const uint32_t off = in_x ? (uint32_t)((r0 * ld + c0) * (int64_t)sizeof(T)) : kOutOfBounds;
    uint4 pu[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pu[i] = bload16(rx, in_x ? off + (uint32_t)(i * ld * (int64_t)sizeof(T)) : kOutOfBounds, 0);
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t wd[4] = {pu[i].x, pu[i].y, pu[i].z, pu[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(T) == 2) {
                mb = max(mb, (wd[j] & 0x7FFFu) << 16);
                mb = max(mb, wd[j] & 0x7FFF0000u);
            } else {
                mb = max(mb, wd[j] & 0x7FFFFFFFu);
            }
        }
    }
    const float m = block_max<kResThreads>(__uint_as_float(mb));
    const float amax = exchange_amax<T>(m, rec, polls, x, rows, cols, ld, &s_fail);
    const float g = global_scale_from_amax(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) g_out[0] = g;
    const float s_enc = 1.0f / g;
    fill_recip_table(rtab, s_enc, threadIdx.x, kResThreads);
    pack_train_headers(o, rows, cols, g, (int64_t)blockIdx.x * kResThreads + threadIdx.x,
                       (int64_t)gridDim.x * kResThreads);
    __syncthreads();
    // (the patch stays packed until here)
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(pu[i].x), "+v"(pu[i].y), "+v"(pu[i].z), "+v"(pu[i].w));
    if (live)
        pack_train_patch<T, kVec>(*reinterpret_cast<const T(*)[16][kVec]>(pu), r0, c0, rows, cols, s_enc, rtab, o);
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
    int nq = 0;
    const int rg = given ? 0 : resident_pack_grid(o.n_pad, o.k_pad, rows, ld_x, esize, vec, partials, n_partials, &nq);
    if (rg > 0) {
        AmaxRecord* rec = reinterpret_cast<AmaxRecord*>(partials);
        if (in_dtype == NVFP4_IN_BF16)
            hipLaunchKernelGGL(pack_train_resident_kernel<uint16_t>, dim3(rg), dim3(kResThreads), 0, stream,
                               static_cast<const uint16_t*>(x), rows, cols, ld_x, g, rec, resident_polls(), o, nq);
        else
            hipLaunchKernelGGL(pack_train_resident_kernel<float>, dim3(rg), dim3(kResThreads), 0, stream,
                               static_cast<const float*>(x), rows, cols, ld_x, g, rec, resident_polls(), o, nq);
        return hipGetLastError();
    }
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
    // (both ways, the one-pass encoder pays off only when every workgroup holds four tiles: the encoding
    // after the exchange is twice that of one orientation; 8192 x 4096 bf16 45.2 -> 36.4 us, while
    // 4096 x 4096 on two tiles per workgroup took 25.5 against 25.4 us and 2048 x 4112 23.6 against 21.9)
    int nq = 0;
    int rg = given ? 0 : resident_t_grid(rows, cols, ld_x, in_dtype, x, partials, n_partials, &nq);
    if (nq != kResThreads / kQThreads) rg = 0;
    if (rg > 0) {
        AmaxRecord* rec = reinterpret_cast<AmaxRecord*>(partials);
        if (in_dtype == NVFP4_IN_BF16)
            hipLaunchKernelGGL((quantize_t_resident_kernel<uint16_t, kTBoth>), dim3(rg), dim3(kResThreads), 0, stream,
                               static_cast<const uint16_t*>(x), rows, cols, ld_x, codes_t, scales_t, g, rec,
                               resident_polls(), codes, scales, nq);
        else
            hipLaunchKernelGGL((quantize_t_resident_kernel<float, kTBoth>), dim3(rg), dim3(kResThreads), 0, stream,
                               static_cast<const float*>(x), rows, cols, ld_x, codes_t, scales_t, g, rec,
                               resident_polls(), codes, scales, nq);
        return hipGetLastError();
    }
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
    int rg = given ? 0 : resident_grid(rows, K, ld_x, in_dtype, x, partials, n_partials);
    // With the transform, each block is transformed twice in one pass (for its max, then for its encoding),
    // which pays only with several blocks per thread: measured, 2 per thread (2048 x 4112 bf16) 13.2 us
    // against 12.5 us in two passes, 5 per thread (4096 x 5120) 19.0 against 22.1 us.
    if (rht && rg > 0 && rows * (K / 16) < 4 * (int64_t)rg * kResThreads) rg = 0;
    if (rg > 0) {
        const int polls = resident_polls();
        AmaxRecord* rec = reinterpret_cast<AmaxRecord*>(partials);
        if (in_dtype == NVFP4_IN_BF16) {
            const uint16_t* xb = static_cast<const uint16_t*>(x);
            if (rht)
                hipLaunchKernelGGL((quantize_resident_kernel<uint16_t, true>), dim3(rg), dim3(kResThreads), 0, stream,
                                   xb, rows, K, ld_x, codes, scales, g, rec, polls, signs);
            else
                hipLaunchKernelGGL((quantize_resident_kernel<uint16_t, false>), dim3(rg), dim3(kResThreads), 0,
                                   stream, xb, rows, K, ld_x, codes, scales, g, rec, polls, 0u);
        } else {
            const float* xf = static_cast<const float*>(x);
            if (rht)
                hipLaunchKernelGGL((quantize_resident_kernel<float, true>), dim3(rg), dim3(kResThreads), 0, stream,
                                   xf, rows, K, ld_x, codes, scales, g, rec, polls, signs);
            else
                hipLaunchKernelGGL((quantize_resident_kernel<float, false>), dim3(rg), dim3(kResThreads), 0, stream,
                                   xf, rows, K, ld_x, codes, scales, g, rec, polls, 0u);
        }
        return hipGetLastError();
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
