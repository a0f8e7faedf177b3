// Few-token (M <= 16) NVFP4 products, bound by the weight stream from HBM.
//
// Work split: workgroup (g, s) owns 4 consecutive 16-row weight blocks (one per
// wavefront) and K-slice s (NKSL k-steps of 128).  Every wavefront issues all
// the loads of its weight slice (16 B of codes + 2 B of scales per lane and
// k-step) first, so the grid's whole weight stream is in flight at once.
// Meanwhile the workgroup prepares the activations of its slice exactly once,
// as FP16 values code x scale laid out in LDS in the B-operand order of the
// 16x16x32 matrix instruction, shared by its 4 wavefronts:
//   CODES mode (nvfp4_gemm): decode the caller's activation codes and scales;
//   QUANT mode (nvfp4_linear): quantize the raw activations of the slice (with
//     the tensor's global scale from the amax partials) and decode them; the
//     workgroups of weight group 0 also store the codes and scales they made.
// Each wavefront then decodes its weight registers and accumulates a 16x16
// tile.  The S slices of a weight group are summed by whichever of its
// workgroups arrives last: each writes its partial tile past the caches,
// waits for the stores, and increments the group's counter; the one that draws
// ticket S-1 adds the S partials in slice order 0..S-1 (so the result does not
// depend on arrival order), applies g_x * g_w and stores Y, then clears the
// counter for the next call.  Nothing ever waits on another workgroup.
#include "common.h"

namespace nvfp4 {

constexpr int kSkThreads = kSkWaves * 64;
constexpr int kSkRows = 4 * 16;               // weight rows per workgroup
constexpr int kWriteThrough = 1 | 16;         // sc0|sc1: store/load past the non-coherent caches

template <typename T> struct RawBlock;   // one 16-element activation block, as loaded
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

// Activation-operand LDS offset (bytes) of chunk c of k-step j for token m, lane group kg.
__device__ __forceinline__ int xhat_offset(int j, int c, int m, int kg) {
    return ((j * 4 + c) * 64 + m + 16 * kg) * 16;
}

// Write the two FP16 chunks of one decoded 16-element block (local block kb of the slice, token m).
__device__ __forceinline__ void put_block(uint8_t* lds, int kb, int m, const half8& lo, const half8& hi) {
    const int j = kb >> 3, b8 = kb & 7, kg = b8 >> 1, c0 = (b8 & 1) * 2;
    *reinterpret_cast<half8*>(lds + xhat_offset(j, c0, m, kg)) = lo;
    *reinterpret_cast<half8*>(lds + xhat_offset(j, c0 + 1, m, kg)) = hi;
}

template <typename T, int NKSL, bool QUANT>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(
    int M, int64_t K, const T* __restrict__ x, int64_t ld_x, const float* __restrict__ amax_partials,
    int n_partials, float* __restrict__ g_x, int g_given, uint8_t* __restrict__ x_codes,
    uint8_t* __restrict__ x_scales, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ colscale, int64_t N, int64_t n_pad, float* __restrict__ y, int64_t ld_y,
    uint32_t* __restrict__ counters, float* __restrict__ partials, int S) {
    __shared__ __attribute__((aligned(16))) uint8_t xhat[NKSL * 4 * 64 * 16];
    __shared__ float s_red[kSkWaves];
    __shared__ int s_last;

    const int grp = blockIdx.x / S, slice = blockIdx.x - grp * S;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int KS = (int)(K / kPackK);
    const int r16 = lane & 15, kg = lane >> 4;
    const int nb = grp * 4 + wave;                 // this wavefront's 16-row weight block
    const int ks0 = slice * NKSL;

    // Loads complete in issue order, so everything the activation preparation
    // needs is requested before the weight stream; preparing the slice then
    // waits only for these, while the weights keep streaming.
    constexpr int kSliceBlocks = NKSL * 8;          // 16-element blocks per token in the slice
    constexpr int kBPT = (16 * kSliceBlocks + kSkThreads - 1) / kSkThreads;
    RawBlock<T> raw[QUANT ? kBPT : 1];
    uint2 cw[QUANT ? 1 : kBPT];
    uint32_t sw[QUANT ? 1 : kBPT];
#pragma unroll
    for (int u = 0; u < kBPT; ++u) {
        const int b = threadIdx.x + u * kSkThreads;
        const int m = b / kSliceBlocks, kb = b - m * kSliceBlocks;
        if (b < 16 * kSliceBlocks && m < M) {
            if constexpr (QUANT) {
                const uint4* src = reinterpret_cast<const uint4*>(x + m * ld_x + (int64_t)(ks0 * 8 + kb) * 16);
#pragma unroll
                for (int q = 0; q < (int)(sizeof(raw[u].v) / 16); ++q) raw[u].v[q] = src[q];
            } else {
                const int64_t blk = (int64_t)m * (K / 16) + ks0 * 8 + kb;
                cw[u] = *reinterpret_cast<const uint2*>(x_codes + blk * 8);
                sw[u] = x_scales[blk];
            }
        }
    }
    float part = 0.0f, g_in = 0.0f;
    if (QUANT && !g_given) {
        for (int i = threadIdx.x; i < n_partials; i += kSkThreads) part = fmaxf(part, amax_partials[i]);
    } else {
        g_in = g_x[0];
    }

    // the weight slice: every load of the wavefront in flight
    const rsrc_t rwc = make_rsrc(w_codes, (uint64_t)n_pad * K / 2);
    const rsrc_t rws = make_rsrc(w_scales, (uint64_t)n_pad * K / 16);
    const uint32_t wc_off = (uint32_t)nb * KS * 1024 + kg * 256 + r16 * 16;
    const uint32_t ws_off = (uint32_t)nb * KS * 128 + r16 * 8 + kg * 2;
    uint4 wv[NKSL];
    uint32_t wsv[NKSL];
#pragma unroll
    for (int j = 0; j < NKSL; ++j) {
        wv[j] = bload16(rwc, wc_off, (uint32_t)(ks0 + j) * 1024);
        wsv[j] = bload2(rws, ws_off, (uint32_t)(ks0 + j) * 128);
    }
    __builtin_amdgcn_sched_barrier(0);

    // the activations of the slice, once per workgroup, as exact FP16 in LDS
    float gx = g_in;
    if (QUANT && !g_given) {
        part = wave_max(part);
        if (lane == 0) s_red[wave] = part;
        __syncthreads();
        float a = s_red[0];
#pragma unroll
        for (int i = 1; i < kSkWaves; ++i) a = fmaxf(a, s_red[i]);
        gx = global_scale_from_amax(a);
        if (blockIdx.x == 0 && threadIdx.x == 0) g_x[0] = gx;
    }
#pragma unroll
    for (int u = 0; u < kBPT; ++u) {
        const int b = threadIdx.x + u * kSkThreads;
        const int m = b / kSliceBlocks, kb = b - m * kSliceBlocks;
        if (b < 16 * kSliceBlocks) {
            half8 lo = {}, hi = {};
            if (m < M) {
                if constexpr (QUANT) {
                    float v[16];
                    widen(raw[u], v);
                    uint32_t c_lo, c_hi, S8;
                    encode_block(v, 1.0f / gx, c_lo, c_hi, S8);
                    const _Float16 s16 = e4m3_to_f16(S8);
                    lo = decode8(c_lo, s16);
                    hi = decode8(c_hi, s16);
                    if (grp == 0) {   // one workgroup per slice stores the activations' NVFP4 encoding
                        const int64_t blk = (int64_t)m * (K / 16) + ks0 * 8 + kb;
                        *reinterpret_cast<uint2*>(x_codes + blk * 8) = make_uint2(c_lo, c_hi);
                        x_scales[blk] = (uint8_t)S8;
                    }
                } else {
                    const _Float16 s16 = e4m3_to_f16(sw[u]);
                    lo = decode8(cw[u].x, s16);
                    hi = decode8(cw[u].y, s16);
                }
            }
            put_block(xhat, kb, m, lo, hi);
        }
    }
    __syncthreads();

    // 3. weight decode + 16x16x32 products over the slice
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NKSL; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const half8 a = decode8(word_of(wv[j], c), scale_byte(wsv[j], c >> 1));
            const half8 b = *reinterpret_cast<const half8*>(xhat + xhat_offset(j, c, r16, kg));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
        }
    }

    // 4. combine the S slices of this weight group (lane holds rows 4*kg..4*kg+3 of block nb, token r16)
    const int64_t n_base = (int64_t)nb * 16 + kg * 4;
    if (S == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n_base + r;
            if (r16 < M && n < N) y[(int64_t)r16 * ld_y + n] = acc[r] * (gx * colscale[n]);
        }
        return;
    }
    const rsrc_t rpart = make_rsrc(partials, (uint64_t)gridDim.x * kSkThreads * 16);
    const uint32_t poff = (uint32_t)threadIdx.x * 16;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc), rpart, (int)poff,
                                           (int)(blockIdx.x * kSkThreads * 16), kWriteThrough);
    __builtin_amdgcn_s_waitcnt(0);                  // the partial has reached the coherent level
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t ticket = __hip_atomic_fetch_add(&counters[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = ticket == (uint32_t)(S - 1);
        if (last) __hip_atomic_store(&counters[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    float4v sum = {0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < S; ++t) {
        const float4v p = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rpart, (int)poff, (int)((grp * S + t) * kSkThreads * 16),
                                                           kWriteThrough));
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[r] += p[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t n = n_base + r;
        if (r16 < M && n < N) y[(int64_t)r16 * ld_y + n] = sum[r] * (gx * colscale[n]);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static const int kNkslOptions[] = {10, 8, 16, 5, 4, 2, 1};

// K-slice length (k-steps) and slice count for a weight: the longest slice that
// still gives >= 256 workgroups (one per CU), else the most workgroups possible.
static void skinny_split(const nvfp4_weight_desc& d, int* nksl, int* S) {
    const int KS = (int)(d.k / kPackK);
    const int64_t groups = d.n_padded / kSkRows;
    int best = 0, best_S = 0;
    for (int opt : kNkslOptions) {
        if (KS % opt != 0) continue;
        const int s = KS / opt;
        if (groups * s >= 256) { *nksl = opt; *S = s; return; }
        if (best == 0 || s > best_S) { best = opt; best_S = s; }
    }
    *nksl = best;
    *S = best_S;
}

bool skinny_applies(int64_t M, const nvfp4_weight_desc& d) {
    if (M < 1 || M > kSkinnyM) return false;
    int nksl = 0, S = 0;
    skinny_split(d, &nksl, &S);
    return nksl > 0;
}

size_t skinny_workspace_bytes(const nvfp4_weight_desc& d) {
    int nksl = 0, S = 0;
    skinny_split(d, &nksl, &S);
    const size_t groups = (size_t)(d.n_padded / kSkRows);
    const size_t counters = (groups * 4 + 255) / 256 * 256;
    return counters + groups * (size_t)S * kSkThreads * 16;
}

template <typename T, bool QUANT>
static hipError_t launch_nksl(int nksl, dim3 grid, hipStream_t stream, int M, int64_t K, const T* x, int64_t ld_x,
                              const float* amax_partials, int n_partials, float* g_x, int g_given, uint8_t* x_codes,
                              uint8_t* x_scales, const uint8_t* wc, const uint8_t* wsc, const float* cs, int64_t N,
                              int64_t n_pad, float* y, int64_t ld_y, uint32_t* counters, float* partials, int S) {
#define NVFP4_SK(NK)                                                                                              \
    case NK:                                                                                                      \
        hipLaunchKernelGGL((skinny_kernel<T, NK, QUANT>), grid, dim3(kSkThreads), 0, stream, M, K, x, ld_x,      \
                           amax_partials, n_partials, g_x, g_given, x_codes, x_scales, wc, wsc, cs, N, n_pad, y, \
                           ld_y, counters, partials, S);                                                          \
        break;
    switch (nksl) {
        NVFP4_SK(1)
        NVFP4_SK(2)
        NVFP4_SK(4)
        NVFP4_SK(5)
        NVFP4_SK(8)
        NVFP4_SK(10)
        NVFP4_SK(16)
        default: return hipErrorInvalidValue;
    }
#undef NVFP4_SK
    return hipGetLastError();
}

hipError_t launch_skinny(int64_t M, const void* x, int in_dtype, int64_t ld_x, const float* amax_partials,
                         int n_partials, float* g_x, int g_mode, uint8_t* x_codes, uint8_t* x_scales, bool quantize,
                         const nvfp4_weight_desc& d, float* y, int64_t ld_y, void* ws, hipStream_t stream) {
    int nksl = 0, S = 0;
    skinny_split(d, &nksl, &S);
    const int64_t groups = d.n_padded / kSkRows;
    const uint8_t* blob = static_cast<const uint8_t*>(d.blob);
    const uint8_t* wc = blob + d.codes_offset;
    const uint8_t* wsc = blob + d.scales_offset;
    const float* cs = reinterpret_cast<const float*>(blob + d.colscale_offset);
    uint32_t* counters = static_cast<uint32_t*>(ws);
    float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (groups * 4 + 255) / 256 * 256);
    const dim3 grid((unsigned)(groups * S));
    const int given = g_mode == NVFP4_G_GIVEN;
    if (!quantize)
        return launch_nksl<uint16_t, false>(nksl, grid, stream, (int)M, d.k, nullptr, 0, nullptr, 0, g_x, 1, x_codes,
                                            x_scales, wc, wsc, cs, d.n, d.n_padded, y, ld_y, counters, partials, S);
    if (in_dtype == NVFP4_IN_BF16)
        return launch_nksl<uint16_t, true>(nksl, grid, stream, (int)M, d.k, static_cast<const uint16_t*>(x), ld_x,
                                           amax_partials, n_partials, g_x, given, x_codes, x_scales, wc, wsc, cs, d.n,
                                           d.n_padded, y, ld_y, counters, partials, S);
    return launch_nksl<float, true>(nksl, grid, stream, (int)M, d.k, static_cast<const float*>(x), ld_x,
                                    amax_partials, n_partials, g_x, given, x_codes, x_scales, wc, wsc, cs, d.n,
                                    d.n_padded, y, ld_y, counters, partials, S);
}

}  // namespace nvfp4
