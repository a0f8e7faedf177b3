// Few-token (1 <= M <= 16) NVFP4 products, bound by the weight stream from HBM.
//
// Work split.  One product workgroup per RB 16-row blocks of the packed
// weight, over all of K: W wavefronts, wavefront w owns the k-steps
// [w*NKW, (w+1)*NKW) of every one of its blocks.  Each wavefront issues all its
// weight loads at the start and decodes them to FP16 registers as they arrive,
// so nothing stands in front of the weight stream.  Per block the W partial
// 16x16 tiles are added through LDS in wavefront order (a fixed order: the
// result never depends on timing, nor on RB) and the workgroup writes the
// block's 16 columns of Y.  No workgroup adds another's partials.  RB = 2
// when K <= 5120 (NKW <= 5, the two blocks' decoded weights then fit two
// wavefronts per SIMD): each activation fragment then serves 32 weight rows,
// which halves the activation reads from the L2, and every workgroup has its
// compute unit to itself (the decode layer: fused step 11.2 -> 8.4 us,
// product alone 9.5 -> 8.0 us); RB = 1 otherwise.
//
// Activations are the B operand of the 16x16x32 instruction, read straight
// from the canonical encoding: lane (token t, lane group kg) needs, per k-step
// ks, the code bytes [ks*64 + 16kg, +16) of token t's row (the 32 elements the
// weight lane (row, kg) holds) and the scales [ks*8 + 2kg, +2); rows t >= M
// read zero through the buffer bounds.
//   nvfp4_gemm: the encoding is an input, loaded together with the weights.
//   nvfp4_linear: the encoding is made in the same launch, once per XCD.
//
// Encoding inside one XCD.  Each XCD has its own L2, and a hand-over between
// workgroups of one XCD goes through that L2 (a few hundred ns), while one
// between XCDs goes to memory (microseconds under a full weight stream).  So
// every XCD encodes the activations itself, into a copy in the product's
// order in the workspace (the bytes are the same whoever writes them), and its
// product workgroups wait only for their own XCD's encoders:
//   - workgroups 0 .. 8E-1 are encoders: workgroup i encodes share i / 8 for
//     the XCD it runs on (the hardware hands out workgroups round-robin over
//     the XCDs, from an XCD that depends on earlier launches, so any 8
//     consecutive workgroups cover the 8 XCDs once each);
//   - the E encoders of an XCD each reduce max|x| over 1/E of the tensor and
//     exchange the partial maxima through the L2 (or take the given g), then
//     encode their 1/E of the 16-element blocks into the product-order copy
//     and raise their `ready` flag;
//   - a product workgroup decodes its weights, waits for the E flags of its
//     XCD and then loads the product-order copy past its L1; after its
//     products it writes its share of the k-steps (the product workgroups
//     split them) of the canonical encoding, the call's output, from those
//     registers, so each output byte is written once rather than once per XCD.
// Every workgroup reads the XCD it runs on from the XCC_ID hardware register.
// One whose wait exceeds a bound (its XCD lacks an encoder share, if the
// hand-out ever differs from the above) encodes all the blocks itself instead
// (the same bytes), so no result depends on where workgroups run or on
// another one being resident.
// The hand-over uses no atomics: each encoder owns its words and writes them
// with plain stores, which land in its XCD's L2 (after a wait for the data
// they publish), and readers poll them with loads past their L1.  A flag holds
// a tag of the launch (dispatch id and queue), so a flag left by an earlier
// launch reads as not raised: nothing is reset after a launch and no
// workgroup waits for another to finish.
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "launch_tag.h"

#pragma clang fp contract(off)

namespace nvfp4 {

constexpr int kXcds = 8;                 // MI355X
constexpr int kEncPerXcd = 8;            // encoder workgroups per XCD (nvfp4_linear); with 16 the 448
                                         // workgroups of the decode layer no longer all fit at once
constexpr int kWaves = 8;                // wavefronts per product workgroup (fewer when K is short)
constexpr int kMaxNkw = 8;               // k-steps per wavefront: K <= 8 * 8 * 128
constexpr int kEncBlocksPerThread = 2;   // blocks an encoder thread holds: 8 * 512 * 2 >= 16 * 8192 / 16
constexpr int kDefaultPolls = 1 << 15;   // polls (each after a short sleep) before encoding locally
constexpr uint32_t kDeadOffset = 0x80000000u;   // scalar offset past every buffer: the load reads zero
// Cache policy of the hand-over loads: sc1.  Measured on MI355X between two
// CUs of one XCD: loads with sc1 (or nt) see another CU's plain store within
// 0.05-0.3 us (served by the XCD's L2), while plain or sc0 loads keep
// returning the stale value even after an L1 invalidate.
constexpr int kPastL1 = 16;
// Cache policy of the weight loads: nontemporal (every weight byte is read
// once per launch; measured on the decode layer: 8.39 -> 8.09 us per step).
constexpr int kStreamed = 2;

// Per-XCD words of the workspace (256 bytes): per encoder e, a 16-byte record
// of its partial max|x| {tag low, tag high, max bits, check} (one store; the
// check word, tag low ^ tag high ^ max ^ a constant, rejects a record read
// while half written), and the launch tag once its blocks are encoded.
struct XcdWords {
    uint4 amax_rec[kEncPerXcd];
    uint64_t ready_flag[kEncPerXcd];
    uint32_t pad[16];
};
constexpr uint32_t kRecCheck = 0x5A17C3E5u;
static_assert(sizeof(XcdWords) == 256, "two 128-byte lines per XCD");
static_assert(kXcds * sizeof(XcdWords) <= kSkinnyCounterBytes, "the workspace holds every XCD's words");

// Wait for this wavefront's LDS accesses, then the workgroup barrier (outstanding
// global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left at their maxima
    __builtin_amdgcn_s_barrier();
}

// The XCD this wavefront runs on.
__device__ __forceinline__ uint32_t hw_xcc_id() {
    return (uint32_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 0xFu;   // hwreg(HW_REG_XCC_ID, 0, 4)
}

// Raise this encoder's flag: the data it publishes (stored by every thread of
// the workgroup before the barrier that precedes this call) is in the L2.
__device__ __forceinline__ void raise_flag(uint64_t* flag, uint64_t tag) {
    __builtin_amdgcn_s_waitcnt(0);
    *reinterpret_cast<volatile uint64_t*>(flag) = tag;
}

// Poll the kEncPerXcd flags from the L2 until all hold `tag`, at most `polls`
// times.  True when they did.
__device__ __forceinline__ bool wait_flags(const uint64_t* flags, uint64_t tag, int polls) {
    static_assert(kEncPerXcd % 2 == 0, "two flags per 16-byte load");
    const rsrc_t r = make_rsrc(flags, kEncPerXcd * 8);
    for (int i = 0; i < polls; ++i) {
        bool all = true;
#pragma unroll
        for (int q = 0; q < kEncPerXcd / 2; ++q) {
            const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * q, 0, kPastL1));
            all = all && ((uint64_t)v.y << 32 | v.x) == tag && ((uint64_t)v.w << 32 | v.z) == tag;
        }
        if (all) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// max over the workgroup of a non-negative 32-bit key; every thread gets it.
__device__ __forceinline__ uint32_t wg_max_u32(uint32_t v, uint32_t* s_red, int nwaves) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    lds_barrier();
    uint32_t r = 0;
    for (int i = 0; i < nwaves; ++i) r = max(r, s_red[i]);
    lds_barrier();   // s_red may be reused
    return r;
}

struct SkinnyParams {
    int M;
    int KS;                  // k-steps of 128 elements
    int64_t K;
    const void* x;           // raw activations (nvfp4_linear)
    int64_t ld_x;
    float* g_x;
    int g_given;
    uint8_t* x_codes;        // canonical encoding (input of nvfp4_gemm, output of nvfp4_linear)
    uint8_t* x_scales;
    const uint8_t* wc;       // packed weight codes, scales, column scales
    const uint8_t* wsc;
    const float* cs;
    int64_t N, n_pad;
    float* y;
    int64_t ld_y;
    XcdWords* xw;            // workspace: one XcdWords per XCD (nvfp4_linear)
    uint8_t* xf;             // workspace: the encoding again, in the product's order (nvfp4_linear)
    int n_enc;               // encoder workgroups (kXcds * kEncPerXcd, or 0)
    int polls;
    uint32_t kb_magic;       // ceil(2^32 / (K/16)): b / (K/16) = umulhi(b, kb_magic) for every block index b
    Epilogue gp;
};

// ---------------------------------------------------------------------------
// Encoding the activations (whole workgroup).
// ---------------------------------------------------------------------------

// Bits of max |v| over one raw block (finite values order like their bit patterns).
template <typename T>
__device__ __forceinline__ uint32_t raw_block_amax_bits(const RawBlock<T>& r) {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < (int)(sizeof(RawBlock<T>) / 16); ++q) {
        const uint32_t w[4] = {r.v[q].x, r.v[q].y, r.v[q].z, r.v[q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 2) {
                m = max(m, (w[i] & 0x7FFFu) << 16);
                m = max(m, w[i] & 0x7FFF0000u);
            } else {
                m = max(m, w[i] & 0x7FFFFFFFu);
            }
        }
    }
    return m;
}

// Raw block b (token b / (K/16), block b % (K/16) of its row); zeros from nblk on.
template <typename T>
__device__ __forceinline__ RawBlock<T> load_raw_block(const SkinnyParams& p, const rsrc_t& rx, uint32_t b,
                                                      uint32_t nblk) {
    const uint32_t kb_per_row = (uint32_t)(p.K / 16);
    const uint32_t t = __umulhi(b, p.kb_magic), kb = b - t * kb_per_row;
    const uint32_t off = b < nblk ? (uint32_t)((int64_t)t * p.ld_x * sizeof(T) + (int64_t)kb * 16 * sizeof(T))
                                  : kOutOfBounds;
    RawBlock<T> raw;
#pragma unroll
    for (int q = 0; q < (int)(sizeof(RawBlock<T>) / 16); ++q)
        raw.v[q] = bload16(rx, b < nblk ? off + (uint32_t)q * 16 : kOutOfBounds, 0);
    return raw;
}

// One encoded block: its 8 code bytes and its scale byte.
struct CodedBlock {
    uint32_t lo, hi, S;
};
template <typename T>
__device__ __forceinline__ CodedBlock encode_raw_block(const RawBlock<T>& raw, float s_enc, const float* rtab) {
    float v[16];
    widen(raw, v);
    CodedBlock c;
    encode_block(v, block_amax(v), s_enc, rtab, c.lo, c.hi, c.S);
    return c;
}
// Block b into the canonical encoding (the call's output).
__device__ __forceinline__ void store_canonical(const SkinnyParams& p, uint32_t b, const CodedBlock& c) {
    *reinterpret_cast<uint2*>(p.x_codes + (size_t)b * 8) = make_uint2(c.lo, c.hi);
    p.x_scales[b] = (uint8_t)c.S;
}
// Block b into the product-order copy: block kb of token t goes to k-step
// kb / 8, slot kb % 8 of that token's 64 code bytes (and 8 scale bytes).
__device__ __forceinline__ void store_product_order(const SkinnyParams& p, uint32_t b, const CodedBlock& c) {
    const uint32_t kb_per_row = (uint32_t)(p.K / 16), t = __umulhi(b, p.kb_magic), kb = b - t * kb_per_row;
    const uint32_t ks = kb >> 3, j = kb & 7;
    *reinterpret_cast<uint2*>(p.xf + ks * 1024 + t * 64 + j * 8) = make_uint2(c.lo, c.hi);
    p.xf[(uint32_t)p.KS * 1024 + ks * 128 + t * 8 + j] = (uint8_t)c.S;
}

// g from max|x| over the whole tensor, by one workgroup, one block in flight
// per thread (the slow paths: they must not raise the kernel's registers above
// those of the usual path).
template <typename T>
__device__ float g_here(const SkinnyParams& p, const rsrc_t& rx, uint32_t nblk, uint32_t* s_red, int nthreads) {
    uint32_t m = 0;
    for (uint32_t b = threadIdx.x; b < nblk; b += (uint32_t)nthreads)
        m = max(m, raw_block_amax_bits<T>(load_raw_block<T>(p, rx, b, nblk)));
    return global_scale_from_amax(__uint_as_float(wg_max_u32(m, s_red, nthreads >> 6)));
}

// The whole encoding by one workgroup (the local path): max|x| over the
// tensor (unless g is given), then every block.  Every thread's stores are
// complete on return.
template <typename T>
__device__ float encode_all_here(const SkinnyParams& p, uint32_t* s_red, float* rtab, int nthreads) {
    const uint32_t nblk = (uint32_t)(p.M * (p.K / 16));
    const rsrc_t rx = make_rsrc(p.x, (uint64_t)p.M * p.ld_x * sizeof(T));
    float g;
    if (p.g_given) {
        g = p.g_x[0];
    } else {
        g = g_here<T>(p, rx, nblk, s_red, nthreads);
        if (threadIdx.x == 0) p.g_x[0] = g;
    }
    const float s_enc = 1.0f / g;
    fill_recip_table(rtab, s_enc, threadIdx.x, nthreads);
    lds_barrier();
    for (uint32_t b = threadIdx.x; b < nblk; b += (uint32_t)nthreads)
    {
        const CodedBlock c = encode_raw_block<T>(load_raw_block<T>(p, rx, b, nblk), s_enc, rtab);
        store_canonical(p, b, c);
        store_product_order(p, b, c);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are done
    lds_barrier();
    return g;
}

// Encoder e of XCD `xw`: its 1/E of the blocks, held in registers from the
// start; the XCD's amax from the E partial maxima (or the given g; or, if the
// exchange does not complete within the bound, from the whole tensor read
// here); then g and its blocks in the product's order, and its `ready` flag.
template <typename T>
__device__ void run_encoder(const SkinnyParams& p, uint32_t e, XcdWords* xw, uint64_t tag, uint32_t* s_red,
                            float* rtab, float* s_g, int nthreads) {
    const uint32_t nblk = (uint32_t)(p.M * (p.K / 16));
    const uint32_t per = (nblk + kEncPerXcd - 1) / kEncPerXcd;
    const uint32_t b0 = min(nblk, e * per), b1 = min(nblk, b0 + per);
    const rsrc_t rx = make_rsrc(p.x, (uint64_t)p.M * p.ld_x * sizeof(T));
    RawBlock<T> raw[kEncBlocksPerThread];
#pragma unroll
    for (int j = 0; j < kEncBlocksPerThread; ++j)
        raw[j] = load_raw_block<T>(p, rx, b0 + threadIdx.x + j * nthreads, b1);

    if (p.g_given) {
        if (threadIdx.x == 0) *s_g = p.g_x[0];
    } else {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < kEncBlocksPerThread; ++j) m = max(m, raw_block_amax_bits<T>(raw[j]));
        m = wg_max_u32(m, s_red, nthreads >> 6);
        if (threadIdx.x == 0) {
            const uint32_t lo = (uint32_t)tag, hi = (uint32_t)(tag >> 32);
            xw->amax_rec[e] = make_uint4(lo, hi, m, lo ^ hi ^ m ^ kRecCheck);
            // poll the E records from the L2 until all carry this launch's tag and a valid check
            const rsrc_t rr = make_rsrc(xw->amax_rec, sizeof(xw->amax_rec));
            bool all = false;
            uint32_t amax = 0;
            for (int i = 0; i < p.polls && !all; ++i) {
                all = true;
                amax = 0;
#pragma unroll
                for (int k = 0; k < kEncPerXcd; ++k) {
                    const uint4 r = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, 16 * k, 0,
                                                                                                   kPastL1));
                    all = all && r.x == lo && r.y == hi && r.w == (lo ^ hi ^ r.z ^ kRecCheck);
                    amax = max(amax, r.z);
                }
                if (!all) __builtin_amdgcn_s_sleep(1);
            }
            *s_g = all ? global_scale_from_amax(__uint_as_float(amax)) : -1.0f;
        }
    }
    lds_barrier();
    float g = *s_g;
    if (g < 0.0f) g = g_here<T>(p, rx, nblk, s_red, nthreads);   // (uniform: every thread read the same word)
    // g for this XCD's product workgroups (they read it after the flags; every XCD writes the same value)
    if (!p.g_given && e == 0 && threadIdx.x == 0) p.g_x[0] = g;
    const float s_enc = 1.0f / g;
    fill_recip_table(rtab, s_enc, threadIdx.x, nthreads);
    lds_barrier();
    CodedBlock c[kEncBlocksPerThread];
#pragma unroll
    for (int j = 0; j < kEncBlocksPerThread; ++j) {
        const uint32_t b = b0 + threadIdx.x + j * nthreads;
        c[j] = encode_raw_block<T>(raw[j], s_enc, rtab);
        if (b < b1) store_product_order(p, b, c[j]);
    }
    __builtin_amdgcn_s_waitcnt(0);   // every thread's product-order blocks (and g) are in the L2
    lds_barrier();
    if (threadIdx.x == 0) raise_flag(&xw->ready_flag[e], tag);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <typename T, int NKW, bool ENC, bool EPI, int RB>
__global__ __launch_bounds__(kWaves * 64) void skinny_kernel(SkinnyParams p) {
    __shared__ __attribute__((aligned(16))) float4v red[RB][kWaves][64];
    __shared__ uint32_t s_red[kWaves];
    __shared__ float rtab[ENC ? 128 : 1];
    __shared__ float s_g;
    __shared__ int s_local;

    const int nthreads = (int)blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r16 = lane & 15, kg = lane >> 4;

    uint64_t tag = 0;
    uint32_t xcd = 0;
    bool xcd_ok = false;
    if constexpr (ENC) {
        tag = launch_tag();
        xcd = hw_xcc_id();
        xcd_ok = xcd < (uint32_t)kXcds;
        if ((int)blockIdx.x < p.n_enc) {   // encoder workgroup: share blockIdx / 8 of its XCD
            if (xcd_ok) run_encoder<T>(p, (uint32_t)blockIdx.x / kXcds, p.xw + xcd, tag, s_red, rtab, &s_g, nthreads);
            return;
        }
    }
    // this workgroup's RB 16-row weight blocks: nb*RB .. nb*RB + RB-1 (those past
    // the weight's row blocks are neither loaded nor stored)
    const int nb = (int)blockIdx.x - (ENC ? p.n_enc : 0);
    const int row_blocks = (int)((p.N + 15) / 16);
    const int ks0 = wave * NKW;
    // k-steps [cks0, cks1) of the call's output encoding are this workgroup's to
    // write (the G product workgroups split the KS k-steps; each is written once)
    int cks0 = 0, cks1 = 0;
    if constexpr (ENC) {
        const int G = (int)gridDim.x - p.n_enc;
        cks0 = nb * p.KS / G;
        cks1 = (nb + 1) * p.KS / G;
    }

    // Weights first: all NKW k-steps of this wavefront (k-steps past K read zero).
    const rsrc_t rwc = make_rsrc(p.wc, (uint64_t)p.n_pad * p.K / 2);
    const rsrc_t rws = make_rsrc(p.wsc, (uint64_t)p.n_pad * p.K / 16);
    // (lane part in the vector offset, block and k-step in the scalar one: a dead
    // k-step's scalar offset lies past the buffer, and the sum stays below 2^32)
    const uint32_t wc_lane = kg * 256 + r16 * 16, ws_lane = r16 * 8 + kg * 2;
    uint4 wv[RB][NKW];
    uint32_t wsv[RB][NKW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int blk = nb * RB + rb;
        const uint32_t wc_blk = (uint32_t)blk * p.KS * 1024, ws_blk = (uint32_t)blk * p.KS * 128;
#pragma unroll
        for (int j = 0; j < NKW; ++j) {
            const int ks = ks0 + j;
            const bool live = ks < p.KS && blk < row_blocks;   // (wavefront-uniform)
            const uint32_t oc = live ? wc_blk + (uint32_t)ks * 1024 : kDeadOffset;
            const uint32_t os = live ? ws_blk + (uint32_t)ks * 128 : kDeadOffset;
            wv[rb][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rwc, (int)wc_lane, (int)oc,
                                                                                          kStreamed));
            wsv[rb][j] = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rws, (int)ws_lane, (int)os, kStreamed);
        }
    }
    const rsrc_t rcs = make_rsrc(p.cs, (uint64_t)p.n_pad * 4);
    float4v csv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        csv[rb] = __builtin_bit_cast(float4v, bload16(rcs, (uint32_t)((nb * RB + rb) * 16 + kg * 4) * 4, 0));

    // Activation operand: token r16's codes and scales for this wavefront's
    // k-steps (whole offset per lane, scalar offset 0: tokens >= M and dead
    // k-steps read zero).  Made in this launch, they are read past the L1.
    uint4 xv[NKW];
    uint32_t xsv[NKW];
    // nvfp4_gemm reads the canonical encoding (token t's row at t * K/2), where
    // one load touches 16 rows; the fused kernel reads the product-order copy
    // its encoders wrote (k-step ks: the 16 tokens' 64 code bytes in 1 KB, then
    // their 8 scale bytes in 128 B), where it touches one contiguous span.
    auto load_x = [&](auto aux_tag) {
        constexpr int aux = decltype(aux_tag)::value;
        const bool row = r16 < p.M;
        rsrc_t rxc, rxs;
        uint32_t xc_row, xs_row, xc_ks, xs_ks;
        if constexpr (ENC) {
            rxc = make_rsrc(p.xf, (uint64_t)p.KS * 1024);
            rxs = make_rsrc(p.xf + (size_t)p.KS * 1024, (uint64_t)p.KS * 128);
            xc_row = (uint32_t)r16 * 64 + kg * 16;
            xs_row = (uint32_t)r16 * 8 + kg * 2;
            xc_ks = 1024;
            xs_ks = 128;
        } else {
            rxc = make_rsrc(p.x_codes, (uint64_t)p.M * p.K / 2);
            rxs = make_rsrc(p.x_scales, (uint64_t)p.M * p.K / 16);
            xc_row = (uint32_t)r16 * (uint32_t)(p.K / 2) + kg * 16;
            xs_row = (uint32_t)r16 * (uint32_t)(p.K / 16) + kg * 2;
            xc_ks = 64;
            xs_ks = 8;
        }
#pragma unroll
        for (int j = 0; j < NKW; ++j) {
            const int ks = ks0 + j;
            const bool live = row && ks < p.KS;
            xv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rxc, (int)(live ? xc_row + (uint32_t)ks * xc_ks : kOutOfBounds), 0,
                                                   aux));
            xsv[j] = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                rxs, (int)(live ? xs_row + (uint32_t)ks * xs_ks : kOutOfBounds), 0, aux);
        }
    };
    if constexpr (!ENC) load_x(std::integral_constant<int, 0>{});

    // Decode the weights as they arrive.
    half8 a[RB][NKW][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NKW; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                a[rb][j][c] = decode8(word_of(wv[rb][j], c), scale_byte(wsv[rb][j], c >> 1));
                asm volatile("" : "+v"(a[rb][j][c]));   // decode here, while waiting, not next to its use
            }

    float gx;
    if constexpr (ENC) {
        // Wait for this XCD's encoders (thread 0 polls the L2, the workgroup follows).
        if (threadIdx.x == 0) {
            const bool ok = xcd_ok && wait_flags(p.xw[xcd].ready_flag, tag, p.polls);
            s_local = ok ? 0 : 1;
        }
        lds_barrier();
        if (s_local) {
            gx = encode_all_here<T>(p, s_red, rtab, nthreads);   // the same bytes the encoders would write
        } else {
            const rsrc_t rg = make_rsrc(p.g_x, 4);
            gx = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, 0, 0, kPastL1));
        }
        load_x(std::integral_constant<int, kPastL1>{});
    } else {
        gx = p.g_x[0];
    }

    // 16x16x32 products over this wavefront's k-steps, into two accumulators
    // (chunks 0, 1 and 2, 3 of each k-step) so that consecutive instructions do
    // not wait for each other's results.
    // In the fused kernel each k-step of this workgroup's share of the call's
    // output encoding is stored from the same registers (token r16: code bytes
    // kg*16 .. kg*16+15 of the k-step and its scale bytes 2kg, 2kg+1); a
    // workgroup that encoded locally has written all of it already.
    // (buffer stores: rows r16 >= M fall past the buffers and are dropped)
    if constexpr (ENC) {
        const bool out_enc = !s_local;
        const rsrc_t roc = make_rsrc(p.x_codes, (uint64_t)p.M * p.K / 2);
        const rsrc_t ros = make_rsrc(p.x_scales, (uint64_t)p.M * p.K / 16);
        // (the scale offset is the code offset / 8: r16*K/16 + 2kg)
        const uint32_t oc = (uint32_t)r16 * (uint32_t)(p.K / 2) + kg * 16;
#pragma unroll
        for (int j = 0; j < NKW; ++j) {
            const int ks = ks0 + j;
            if (out_enc && ks >= cks0 && ks < cks1) {   // (workgroup-uniform)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, xv[j]), roc, (int)oc, ks * 64, 0);
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)xsv[j], ros, (int)(oc >> 3), ks * 8, 0);
            }
        }
    }
    // (the activation fragment of a chunk serves every row block)
    float4v acc0[RB], acc1[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc0[rb] = acc1[rb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NKW; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const half8 b = decode8(word_of(xv[j], c), scale_byte(xsv[j], c >> 1));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if (c & 1) acc1[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rb][j][c], b, acc1[rb], 0, 0, 0);
                else acc0[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rb][j][c], b, acc0[rb], 0, 0, 0);
            }
        }
    }

    // Partial tiles summed in wavefront order, row block rb by wavefront rb.
    // Lane holds rows 4kg..4kg+3 of the block for token r16.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) red[rb][wave][lane] = acc0[rb] + acc1[rb];
    lds_barrier();
    const int nw = nthreads >> 6;
    if (r16 >= p.M) return;
    for (int rb = wave; rb < RB; rb += nw) {   // (wavefront-uniform)
        const int blk = nb * RB + rb;
        if (blk >= row_blocks) break;
        float4v sum = red[rb][0][lane];
        for (int w = 1; w < nw; ++w) sum += red[rb][w][lane];
        const int64_t n_base = (int64_t)blk * 16 + kg * 4;
        bool gated = false;   // only the row blocks that hold gate columns take the gated stores
        if constexpr (EPI) gated = gates_touch((int64_t)blk * 16, (int64_t)blk * 16 + 16, p.gp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n_base + r;
            if (n < p.N) {
                float v = sum[r] * (gx * csv[rb][r]);
                if constexpr (EPI) {
                    if (gated) v = gate(v, n, p.gp);
                    store_y(p.y, (int64_t)r16 * p.ld_y + n, v, p.gp);
                } else {
                    p.y[(int64_t)r16 * p.ld_y + n] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

struct SkinnyPlan {
    int waves = 0, nkw = 0;
    bool ok() const { return waves > 0; }
};

// kWaves wavefronts (fewer when K has fewer k-steps), each with ceil(KS / waves) k-steps.
SkinnyPlan plan_for(const nvfp4_weight_desc& d) {
    SkinnyPlan p;
    const int64_t KS = d.k / kPackK;
    if (KS < 1 || KS > (int64_t)kWaves * kMaxNkw) return p;
    p.waves = (int)(KS < kWaves ? KS : kWaves);
    p.nkw = (int)((KS + p.waves - 1) / p.waves);
    return p;
}

// Row blocks per product workgroup: two while both blocks' decoded weights fit
// the registers of two wavefronts per SIMD (NKW <= 5), so that each
// workgroup's activation loads serve 32 weight rows and every workgroup runs
// alone on its compute unit; one otherwise.
template <int NKW, bool ENC>
struct RowBlocks : std::integral_constant<int, NKW <= 5 ? 2 : 1> {};

template <typename T, int NKW, bool ENC>
void launch_one(unsigned blocks, unsigned n_enc, int waves, hipStream_t stream, const SkinnyParams& a, bool epi) {
    constexpr int RB = RowBlocks<NKW, ENC>::value;
    auto kern = epi ? skinny_kernel<T, NKW, ENC, true, RB> : skinny_kernel<T, NKW, ENC, false, RB>;
    hipLaunchKernelGGL(kern, dim3((blocks + RB - 1) / RB + n_enc), dim3(waves * 64), 0, stream, a);
}

template <typename T, bool ENC>
hipError_t launch_nkw(const SkinnyPlan& pl, unsigned blocks, hipStream_t stream, const SkinnyParams& a, bool epi) {
    const unsigned n_enc = (unsigned)a.n_enc;
    switch (pl.nkw) {
        case 1: launch_one<T, 1, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 2: launch_one<T, 2, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 3: launch_one<T, 3, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 4: launch_one<T, 4, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 5: launch_one<T, 5, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 6: launch_one<T, 6, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 7: launch_one<T, 7, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        case 8: launch_one<T, 8, ENC>(blocks, n_enc, pl.waves, stream, a, epi); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool skinny_applies(int64_t M, const nvfp4_weight_desc& d) {
    if (M < 1 || M > kSkinnyM) return false;
    const SkinnyPlan pl = plan_for(d);
    // an encoder thread holds at most kEncBlocksPerThread blocks of its XCD share
    return pl.ok() && (M * (d.k / 16) + kEncPerXcd - 1) / kEncPerXcd <= (int64_t)kEncBlocksPerThread * pl.waves * 64;
}

// The flags, then the product-order copy of the activation encoding (16 token
// slots per k-step: 1 KB of codes and 128 B of scales).
static size_t product_order_bytes(const nvfp4_weight_desc& d) { return (size_t)(d.k / kPackK) * 1152; }
size_t skinny_workspace_bytes(const nvfp4_weight_desc& d) {
    return plan_for(d).ok() ? kSkinnyCounterBytes + (product_order_bytes(d) + 255) / 256 * 256 : 0;
}

hipError_t launch_skinny(int64_t M, const void* x, int in_dtype, int64_t ld_x, float* g_x, int g_mode,
                         uint8_t* x_codes, uint8_t* x_scales, bool quantize, const nvfp4_weight_desc& d, float* y,
                         int64_t ld_y, void* ws, const Epilogue& gp, hipStream_t stream) {
    if (!skinny_applies(M, d)) return hipErrorInvalidValue;
    const SkinnyPlan pl = plan_for(d);
    const uint8_t* blob = static_cast<const uint8_t*>(d.blob);
    SkinnyParams a;
    a.M = (int)M;
    a.KS = (int)(d.k / kPackK);
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
    a.xw = static_cast<XcdWords*>(ws);
    a.xf = quantize ? static_cast<uint8_t*>(ws) + kSkinnyCounterBytes : nullptr;
    a.n_enc = quantize ? kXcds * kEncPerXcd : 0;
    a.gp = gp;
    a.polls = kDefaultPolls;
    // exact for b < 2^32 / (K/16) (ceil(2^32/d)*d - 2^32 < d): every block index here is below 2^17
    a.kb_magic = (uint32_t)(((uint64_t(1) << 32) + (uint64_t)(d.k / 16) - 1) / (uint64_t)(d.k / 16));
    if (const char* e = std::getenv("NVFP4_AMAX_POLLS")) a.polls = std::atoi(e);   // testing the local path
    const bool epi = gp.n_a > 0 || gp.n_b > 0 || gp.out_bf16;
    const unsigned blocks = (unsigned)((d.n + kPackRows - 1) / kPackRows);   // blocks holding real rows
    if (!quantize) return launch_nkw<uint16_t, false>(pl, blocks, stream, a, epi);
    if (in_dtype == NVFP4_IN_BF16) return launch_nkw<uint16_t, true>(pl, blocks, stream, a, epi);
    return launch_nkw<float, true>(pl, blocks, stream, a, epi);
}

}  // namespace nvfp4
