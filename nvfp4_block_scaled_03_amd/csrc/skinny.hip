// Few-token (M <= 16) NVFP4 products, bound by the weight stream from HBM.
//
// Work split.  The weight rows are cut into groups of R 16-row blocks and K
// into S slices of NKSL k-steps (128 elements each).  Workgroup (g, s) has R
// wavefronts; wavefront w owns block g*R + w over slice s.  R, NKSL and S are
// chosen on the host so that the workgroups cover the 256 compute units
// evenly (5120 rows: 64 groups of 5 blocks x 4 slices = 256 workgroups): a
// compute unit's share of the weight stream, not its arithmetic, sets when it
// finishes, so one unit with twice the share finishes twice as late.
//
// Per workgroup.  The activation-side loads are issued first, without
// branches (rows >= M read as zero through the buffer bounds), then the first
// kDepth k-steps of every wavefront's weights.  The activations of the slice
// are prepared once, as exact FP16 values code x scale in LDS, laid out in the
// B-operand order of the 16x16x32 matrix instruction:
//   CODES (nvfp4_gemm): decode the caller's codes and scales;
//   QUANT (nvfp4_linear): quantize the raw activations with the global scale
//     (given, or reduced from the amax partials of the preceding kernel) and
//     decode them; the workgroups of group 0 also store the codes and scales.
// Each wavefront then walks its k-steps: decode the weight chunk, four matrix
// instructions, and issue the loads kDepth k-steps ahead.
//
// Summing the slices.  No workgroup ever waits for one that may not have
// started.  Each workgroup draws a ticket from its group's counter when it
// starts; the one drawing S-1 (the last to start) is the reducer, the others
// store their partial tiles past the caches and finish.  A stored partial is
// negated after -0 is turned into +0, so none of its words is zero; the
// reducer polls each partial until all its words are nonzero, adds the S
// partials in slice order 0..S-1 (its own from registers), so the result does
// not depend on timing, writes Y = sum * g_x * g_w, zeroes the partials it
// read and resets the counter: the workspace is zero again for the next call.
#include <cstdlib>

#include "common.h"

namespace nvfp4 {

constexpr int kWriteThrough = 1 | 16;   // sc0|sc1: store past the non-coherent caches
constexpr int kDepth = 4;               // weight k-steps in flight per wavefront ahead of the math
constexpr int kMaxSlices = 8;           // K-slices per group (the reducer polls at most 7 partials)
constexpr int kSpinLimit = 1 << 20;     // polls before the reducer gives up (a misuse, never a hang)
constexpr int kMaxPre = 10;             // longest slice (bf16 input; 4 for fp32) whose weights are decoded
                                        // ahead of the activations (16 VGPRs per k-step)

constexpr int kAmaxSpin = 1 << 12;      // polls for a peer's slice max before reducing that slice here

// Max over the workgroup (R wavefronts), via LDS scratch of R floats; all threads get it.
template <int R>
__device__ __forceinline__ float block_max_r(float v, float* s_red) {
    v = wave_max(v);
    __syncthreads();   // s_red may still be read from a previous call
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    __syncthreads();
    float a = s_red[0];
#pragma unroll
    for (int i = 1; i < R; ++i) a = fmaxf(a, s_red[i]);
    return a;
}

// Activation-operand LDS offset (bytes) of chunk c of k-step j for token m, lane group kg.
__device__ __forceinline__ int xhat_offset(int j, int c, int m, int kg) {
    return ((j * 4 + c) * 64 + m + 16 * kg) * 16;
}

// Write the two FP16 chunks of one decoded 16-element block (local block kb of the slice, token m);
// a thread without a block (past the slice) writes to the spare 32 bytes at `spare` instead, so the
// preparation has no branch around it.
__device__ __forceinline__ void put_block(uint8_t* lds, int kb, int m, bool valid, int spare, const half8& lo,
                                          const half8& hi) {
    const int j = kb >> 3, b8 = kb & 7, kg = b8 >> 1, c0 = (b8 & 1) * 2;
    const int o0 = valid ? xhat_offset(j, c0, m, kg) : spare;
    const int o1 = valid ? xhat_offset(j, c0 + 1, m, kg) : spare + 16;
    *reinterpret_cast<half8*>(lds + o0) = lo;
    *reinterpret_cast<half8*>(lds + o1) = hi;
}

template <typename T, int NKSL, int R, bool QUANT, bool PRE, bool EPI>
__global__ __launch_bounds__(R * 64) void skinny_kernel(
    int M, int64_t K, const T* __restrict__ x, int64_t ld_x, float* __restrict__ g_x, int g_given,
    uint8_t* __restrict__ x_codes, uint8_t* __restrict__ x_scales, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ colscale, int64_t N, int64_t n_pad,
    float* __restrict__ y, int64_t ld_y, uint32_t* __restrict__ counters, uint32_t* __restrict__ slots,
    float* __restrict__ partials, int S, int amax_polls, Epilogue gp) {
    constexpr int kThreads = R * 64;
    constexpr int kXhatBytes = NKSL * 4 * 64 * 16;
    constexpr int kD = NKSL < kDepth ? NKSL : kDepth;
    __shared__ __attribute__((aligned(16))) uint8_t xhat[kXhatBytes + 32];   // + spare slot
    __shared__ float s_red[R];
    __shared__ float s_slotmax[kMaxSlices];
    __shared__ uint32_t s_ticket;
    __shared__ float rtab[QUANT ? 128 : 1];

    const int grp = blockIdx.x / S, slice = blockIdx.x - grp * S;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int KS = (int)(K / kPackK);
    const int r16 = lane & 15, kg = lane >> 4;
    const int nb = grp * R + wave;                 // this wavefront's 16-row weight block
    const int ks0 = slice * NKSL;

    // Activation-side loads of the slice (branch-free; rows >= M and slots past
    // the slice read as zero through the buffer bounds).
    constexpr int kSliceBlocks = NKSL * 8;          // 16-element blocks per token in the slice
    constexpr int kBPT = (16 * kSliceBlocks + kThreads - 1) / kThreads;
    constexpr int kRawVec = QUANT ? (int)(sizeof(RawBlock<T>) / 16) : 1;
    RawBlock<T> raw[QUANT ? kBPT : 1];
    uint2 cw[QUANT ? 1 : kBPT];
    uint32_t sw[QUANT ? 1 : kBPT];
    auto load_activations = [&]() {
        if constexpr (QUANT) {
            const rsrc_t rx = make_rsrc(x, (uint64_t)M * ld_x * sizeof(T));
#pragma unroll
            for (int u = 0; u < kBPT; ++u) {
                const int b = threadIdx.x + u * kThreads;
                const int m = b / kSliceBlocks, kb = b - m * kSliceBlocks;
                const uint32_t off =
                    m < M ? (uint32_t)(((int64_t)m * ld_x + (int64_t)(ks0 * 8 + kb) * 16) * (int64_t)sizeof(T))
                          : kOutOfBounds;
#pragma unroll
                for (int q = 0; q < kRawVec; ++q) raw[u].v[q] = bload16(rx, off, (uint32_t)q * 16);
            }
        } else {
            const rsrc_t rxc = make_rsrc(x_codes, (uint64_t)M * K / 2);
            const rsrc_t rxs = make_rsrc(x_scales, (uint64_t)M * K / 16);
#pragma unroll
            for (int u = 0; u < kBPT; ++u) {
                const int b = threadIdx.x + u * kThreads;
                const int m = b / kSliceBlocks, kb = b - m * kSliceBlocks;
                const uint32_t blk = (uint32_t)(m * (int)(K / 16) + ks0 * 8 + kb);
                cw[u] = bload8(rxc, m < M ? blk * 8 : kOutOfBounds, 0);
                sw[u] = bload1(rxs, m < M ? blk : kOutOfBounds, 0);
            }
        }
    };

    // Weight slice: kD k-steps in flight ahead of their use.
    const rsrc_t rwc = make_rsrc(w_codes, (uint64_t)n_pad * K / 2);
    const rsrc_t rws = make_rsrc(w_scales, (uint64_t)n_pad * K / 16);
    const uint32_t wc_off = (uint32_t)nb * KS * 1024 + kg * 256 + r16 * 16;
    const uint32_t ws_off = (uint32_t)nb * KS * 128 + r16 * 8 + kg * 2;
    uint4 wv[NKSL];
    uint32_t wsv[NKSL];
    auto load_weights = [&](int j) {
        wv[j] = bload16(rwc, wc_off, (uint32_t)(ks0 + j) * 1024);
        wsv[j] = bload2(rws, ws_off, (uint32_t)(ks0 + j) * 128);
    };
    const rsrc_t rcs = make_rsrc(colscale, (uint64_t)n_pad * 4);
    float4v csv;
    uint32_t ticket = 0;
    // (built with the atomic optimizer off: it would turn this into a wave-wide
    // operation whose result is needed at once, waiting here for every load above)
    auto draw_ticket = [&]() {
        if (S > 1 && threadIdx.x == 0)
            ticket = __hip_atomic_fetch_add(&counters[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    half8 adec[PRE ? NKSL : 1][4];

    // Activations first (loads complete in issue order, so waiting for them
    // leaves the weights in flight), then the weights' first kD k-steps.
    load_activations();
    csv = __builtin_bit_cast(float4v, bload16(rcs, (uint32_t)(nb * 16 + kg * 4) * 4, 0));
#pragma unroll
    for (int j = 0; j < kD; ++j) load_weights(j);
    draw_ticket();
    __builtin_amdgcn_sched_barrier(0);

    // Global scale computed here (nvfp4_linear without a given scale): the S
    // workgroups of a group hold the S slices of the same activations; each
    // publishes its slice's max|x| as soon as its slice is in and collects the
    // others' later.  A slice not published after kAmaxSpin polls is reduced
    // here instead, so no workgroup depends on another one running.
    const bool exchange = QUANT && !g_given;
    uint32_t* gslots = slots + (size_t)grp * S;
    float mine = 0.0f;
    float bam[QUANT ? kBPT : 1];   // max |x| of each of this thread's blocks
    if (exchange) {
        float part = 0.0f;
#pragma unroll
        for (int u = 0; u < (QUANT ? kBPT : 0); ++u) {
            float v[16];
            widen(raw[u], v);
            bam[u] = block_amax(v);
            part = fmaxf(part, bam[u]);
        }
        mine = block_max_r<R>(part, s_red);
        if (S > 1 && threadIdx.x == 0)   // (sign bit set: a published word is never zero)
            __hip_atomic_store(gslots + slice, __float_as_uint(mine) | 0x80000000u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }

    if constexpr (PRE) {
        // Decode the weights to FP16 registers as they arrive, while the slice
        // maxima of the other workgroups travel; only the matrix instructions
        // remain once the activations are prepared.
#pragma unroll
        for (int j = 0; j < NKSL; ++j) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                adec[j][c] = decode8(word_of(wv[j], c), scale_byte(wsv[j], c >> 1));
                asm volatile("" : "+v"(adec[j][c]));   // decode now, not next to its use
            }
            if (j + kD < NKSL) load_weights(j + kD);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    float gx = (QUANT && !g_given) ? 0.0f : g_x[0];
    if (exchange) {
        if (threadIdx.x < (unsigned)S) {
            float got = mine;
            if ((int)threadIdx.x != slice) {
                uint32_t w = 0;
                for (int i = 0; i < amax_polls && w == 0; ++i) {
                    w = __hip_atomic_load(gslots + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (w == 0) __builtin_amdgcn_s_sleep(2);
                }
                got = w != 0 ? __uint_as_float(w & 0x7FFFFFFFu) : -1.0f;
            }
            s_slotmax[threadIdx.x] = got;
        }
        __syncthreads();
        float amax = 0.0f;
        for (int t = 0; t < S; ++t) {
            const float m_t = s_slotmax[t];
            if (m_t >= 0.0f) {
                amax = fmaxf(amax, m_t);
            } else {   // this workgroup reduces slice t itself
                float p = 0.0f;
                for (int b = threadIdx.x; b < M * kSliceBlocks; b += kThreads) {
                    const int m = b / kSliceBlocks, kb = b - m * kSliceBlocks;
                    const T* src = x + (int64_t)m * ld_x + (int64_t)(t * kSliceBlocks + kb) * 16;
                    float v[16];
                    load8(src, v);
                    load8(src + 8, v + 8);
#pragma unroll
                    for (int i = 0; i < 16; ++i) p = fmaxf(p, __builtin_fabsf(v[i]));
                }
                amax = fmaxf(amax, block_max_r<R>(p, s_red));
            }
        }
        gx = global_scale_from_amax(amax);
        if (blockIdx.x == 0 && threadIdx.x == 0) g_x[0] = gx;
    }

    float s_enc = 0.0f;
    if constexpr (QUANT) {
        s_enc = 1.0f / gx;
        fill_recip_table(rtab, s_enc, threadIdx.x, kThreads);
        __syncthreads();
    }

    // The activations of the slice, once per workgroup, as exact FP16 in LDS.
#pragma unroll
    for (int u = 0; u < kBPT; ++u) {
        const int b = threadIdx.x + u * kThreads;
        const int m = b / kSliceBlocks, kb = b - m * kSliceBlocks;
        const bool valid = b < 16 * kSliceBlocks;
        half8 lo, hi;
        if constexpr (QUANT) {
            float v[16];
            widen(raw[u], v);
            uint32_t c_lo, c_hi, S8;
            encode_block(v, exchange ? bam[u] : block_amax(v), s_enc, rtab, c_lo, c_hi, S8);
            const _Float16 s16 = e4m3_to_f16(S8);
            lo = decode8(c_lo, s16);
            hi = decode8(c_hi, s16);
            if (grp == 0 && m < M && valid) {   // one workgroup per slice stores the activations' encoding
                const int64_t blk = (int64_t)m * (K / 16) + ks0 * 8 + kb;
                *reinterpret_cast<uint2*>(x_codes + blk * 8) = make_uint2(c_lo, c_hi);
                x_scales[blk] = (uint8_t)S8;
            }
        } else {
            const _Float16 s16 = e4m3_to_f16(sw[u]);
            lo = decode8(cw[u].x, s16);
            hi = decode8(cw[u].y, s16);
        }
        put_block(xhat, kb, m, valid, kXhatBytes, lo, hi);
    }
    __syncthreads();

    // 16x16x32 products over the slice (weights decoded here, loads kD k-steps
    // ahead, unless already decoded above).
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NKSL; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            half8 a;
            if constexpr (PRE) a = adec[j][c];
            else a = decode8(word_of(wv[j], c), scale_byte(wsv[j], c >> 1));
            const half8 b = *reinterpret_cast<const half8*>(xhat + xhat_offset(j, c, r16, kg));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
        }
        if constexpr (!PRE) {
            if (j + kD < NKSL) load_weights(j + kD);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Lane holds rows 4*kg..4*kg+3 of block nb for token r16.
    const int64_t n_base = (int64_t)nb * 16 + kg * 4;
    bool gated = false;   // only the row blocks that hold gate columns take the gated stores
    if constexpr (EPI) gated = gates_touch((int64_t)nb * 16, (int64_t)nb * 16 + 16, gp);
    if (S == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n_base + r;
            if (r16 < M && n < N) {
                float v = acc[r] * (gx * csv[r]);
                if (EPI && gated) v = gate(v, n, gp);
                if constexpr (EPI)
                    store_y(y, (int64_t)r16 * ld_y + n, v, gp);
                else
                    y[(int64_t)r16 * ld_y + n] = v;
            }
        }
        return;
    }
    if (threadIdx.x == 0) s_ticket = ticket;
    __syncthreads();
    const bool reducer = s_ticket == (uint32_t)(S - 1);
    float4v own;
#pragma unroll
    for (int r = 0; r < 4; ++r) own[r] = acc[r] + 0.0f;   // -0 -> +0
    constexpr int kTile = kThreads * 16;                    // bytes of one partial tile
    const rsrc_t rpart = make_rsrc(partials, (uint64_t)gridDim.x * kTile);
    const uint32_t poff = (uint32_t)threadIdx.x * 16;
    if (!reducer) {
        float4v neg;
#pragma unroll
        for (int r = 0; r < 4; ++r) neg[r] = -own[r];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, neg), rpart, (int)poff,
                                               (int)(blockIdx.x * kTile), kWriteThrough);
        return;
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // Poll every other slice's partial (all loads of a round in flight together).
    float4v pt[kMaxSlices];
    bool ready[kMaxSlices];
#pragma unroll
    for (int t = 0; t < kMaxSlices; ++t) ready[t] = !(t < S && t != slice);
    for (int round = 0;; ++round) {
#pragma unroll
        for (int t = 0; t < kMaxSlices; ++t) {
            if (!ready[t]) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(
                    reinterpret_cast<const uint8_t*>(partials) + (size_t)(grp * S + t) * kTile + poff);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    pt[t][r] = __uint_as_float(
                        __hip_atomic_load(src + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            }
        }
        bool all = true;
#pragma unroll
        for (int t = 0; t < kMaxSlices; ++t) {
            if (!ready[t]) {
                ready[t] = __float_as_uint(pt[t][0]) != 0u && __float_as_uint(pt[t][1]) != 0u &&
                           __float_as_uint(pt[t][2]) != 0u && __float_as_uint(pt[t][3]) != 0u;
                all = all && ready[t];
            }
        }
        if (all || round >= kSpinLimit) break;
        __builtin_amdgcn_s_sleep(2);
    }
    // every member has read the group's slice maxima by now (it stored its partial after)
    if (QUANT && threadIdx.x < (unsigned)S)
        __hip_atomic_store(slots + (size_t)grp * S + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float4v sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kMaxSlices; ++t) {
        if (t < S) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sum[r] += t == slice ? own[r] : -pt[t][r];
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t n = n_base + r;
        if (r16 < M && n < N) {
            float v = sum[r] * (gx * csv[r]);
            if (EPI && gated) v = gate(v, n, gp);
            if constexpr (EPI)
                    store_y(y, (int64_t)r16 * ld_y + n, v, gp);
                else
                    y[(int64_t)r16 * ld_y + n] = v;
        }
    }
    const v4i zero = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < kMaxSlices; ++t) {
        if (t < S && t != slice)
            __builtin_amdgcn_raw_buffer_store_b128(zero, rpart, (int)poff, (int)((grp * S + t) * kTile),
                                                   kWriteThrough);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

struct SkinnyPlan {
    int R = 0, nksl = 0, S = 0;
    int64_t groups = 0;
    bool ok() const { return R > 0; }
    int64_t workgroups() const { return groups * S; }
};

const int kROptions[] = {4, 5, 8};
const int kNkslOptions[] = {16, 10, 8, 5, 4, 2, 1};

// The split whose workgroups spread most evenly over the compute units (each
// unit's share of the weight stream sets its finishing time); ties go to fewer
// slices (less to sum) and then to longer slices.
SkinnyPlan plan_for(const nvfp4_weight_desc& d) {
    SkinnyPlan best;
    double best_eff = -1.0;
    const int KS = (int)(d.k / kPackK);
    const int64_t blocks = d.n_padded / kPackRows;
    for (int R : kROptions) {
        if (blocks % R != 0) continue;
        for (int nksl : kNkslOptions) {
            if (KS % nksl != 0 || KS / nksl > kMaxSlices) continue;
            SkinnyPlan p;
            p.R = R;
            p.nksl = nksl;
            p.S = KS / nksl;
            p.groups = blocks / R;
            const int64_t wgs = p.workgroups();
            const int64_t rounds = (wgs + kComputeUnits - 1) / kComputeUnits;
            const double eff = (double)wgs / (double)(rounds * kComputeUnits);
            const bool better = eff > best_eff + 1e-9 ||
                                (eff > best_eff - 1e-9 && (p.S < best.S || (p.S == best.S && nksl > best.nksl)));
            if (better) {
                best = p;
                best_eff = eff;
            }
        }
    }
    return best;
}

struct SkinnyArgs {
    int M;
    int64_t K;
    const void* x;
    int64_t ld_x;
    float* g_x;
    int g_given;
    uint8_t* x_codes;
    uint8_t* x_scales;
    const uint8_t* wc;
    const uint8_t* wsc;
    const float* cs;
    int64_t N, n_pad;
    float* y;
    int64_t ld_y;
    uint32_t* counters;
    uint32_t* slots;
    float* partials;
    int S;
    int amax_polls;
    Epilogue gp;
    bool epi;
};

template <typename T, int NKSL, int R, bool QUANT>
void launch_one(dim3 grid, hipStream_t stream, const SkinnyArgs& a) {
    constexpr bool kPre = QUANT && NKSL <= kMaxPre / sizeof(T) * 2;
    // the general epilogue (gates, bf16 output) only where asked for: the plain kernel keeps its registers
    auto kern = a.epi ? skinny_kernel<T, NKSL, R, QUANT, kPre, true> : skinny_kernel<T, NKSL, R, QUANT, kPre, false>;
    hipLaunchKernelGGL(kern, grid, dim3(R * 64), 0, stream, a.M, a.K, static_cast<const T*>(a.x), a.ld_x, a.g_x, a.g_given, a.x_codes, a.x_scales,
                       a.wc, a.wsc, a.cs, a.N, a.n_pad, a.y, a.ld_y, a.counters, a.slots, a.partials, a.S,
                       a.amax_polls, a.gp);
}

template <typename T, bool QUANT, int R>
hipError_t launch_nksl(int nksl, dim3 grid, hipStream_t stream, const SkinnyArgs& a) {
    switch (nksl) {
        case 1: launch_one<T, 1, R, QUANT>(grid, stream, a); break;
        case 2: launch_one<T, 2, R, QUANT>(grid, stream, a); break;
        case 4: launch_one<T, 4, R, QUANT>(grid, stream, a); break;
        case 5: launch_one<T, 5, R, QUANT>(grid, stream, a); break;
        case 8: launch_one<T, 8, R, QUANT>(grid, stream, a); break;
        case 10: launch_one<T, 10, R, QUANT>(grid, stream, a); break;
        case 16: launch_one<T, 16, R, QUANT>(grid, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool QUANT>
hipError_t launch_plan(const SkinnyPlan& p, hipStream_t stream, const SkinnyArgs& a) {
    const dim3 grid((unsigned)p.workgroups());
    switch (p.R) {
        case 4: return launch_nksl<T, QUANT, 4>(p.nksl, grid, stream, a);
        case 5: return launch_nksl<T, QUANT, 5>(p.nksl, grid, stream, a);
        case 8: return launch_nksl<T, QUANT, 8>(p.nksl, grid, stream, a);
        default: return hipErrorInvalidValue;
    }
}

// Workspace: one ticket counter per group, S published slice maxima per group,
// then one partial tile per workgroup.
size_t counters_bytes(const SkinnyPlan& p) { return (size_t)((p.groups * (1 + p.S) * 4 + 255) / 256 * 256); }

}  // namespace

bool skinny_applies(int64_t M, const nvfp4_weight_desc& d) {
    if (M < 1 || M > kSkinnyM) return false;
    return plan_for(d).ok();
}

size_t skinny_workspace_bytes(const nvfp4_weight_desc& d) {
    const SkinnyPlan p = plan_for(d);
    if (!p.ok()) return 0;
    return counters_bytes(p) + (size_t)p.workgroups() * (size_t)p.R * 64 * 16;
}

hipError_t launch_skinny(int64_t M, const void* x, int in_dtype, int64_t ld_x, float* g_x, int g_mode,
                         uint8_t* x_codes, uint8_t* x_scales, bool quantize, const nvfp4_weight_desc& d, float* y,
                         int64_t ld_y, void* ws, const Epilogue& gp, hipStream_t stream) {
    const SkinnyPlan p = plan_for(d);
    if (!p.ok()) return hipErrorInvalidValue;
    const uint8_t* blob = static_cast<const uint8_t*>(d.blob);
    SkinnyArgs a;
    a.M = (int)M;
    a.K = d.k;
    a.x = x;
    a.ld_x = ld_x;
    a.g_x = g_x;
    a.g_given = (!quantize || g_mode == NVFP4_G_GIVEN) ? 1 : 0;
    a.x_codes = x_codes;
    a.x_scales = x_scales;
    a.wc = blob + d.codes_offset;
    a.wsc = blob + d.scales_offset;
    a.cs = reinterpret_cast<const float*>(blob + d.colscale_offset);
    a.N = d.n;
    a.n_pad = d.n_padded;
    a.y = y;
    a.ld_y = ld_y;
    a.counters = static_cast<uint32_t*>(ws);
    a.slots = a.counters + p.groups;
    a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + counters_bytes(p));
    a.S = p.S;
    a.gp = gp;
    a.epi = gp.n_a > 0 || gp.n_b > 0 || gp.out_bf16;
    a.amax_polls = kAmaxSpin;
    if (const char* e = std::getenv("NVFP4_AMAX_POLLS")) a.amax_polls = std::atoi(e);   // testing the fallback
    if (!quantize) return launch_plan<uint16_t, false>(p, stream, a);
    if (in_dtype == NVFP4_IN_BF16) return launch_plan<uint16_t, true>(p, stream, a);
    return launch_plan<float, true>(p, stream, a);
}

}  // namespace nvfp4
