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
//
// All operand loads are buffer loads: a scalar resource per tensor, one 32-bit
// per-lane offset, and the per-k-step / per-tile advance in a scalar offset.
// Reads past the end of a tensor return zero, which is how rows beyond M (a
// ragged last tile) contribute nothing without any clamping.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Tiled GEMM: a workgroup of 2x2 wavefronts computes a (2*TM*32) x (2*TN*32)
// output tile; each wavefront a TM x TN grid of 32x32x16 FP16 instructions.
//
// Operands move global -> LDS by buffer loads that write LDS directly (no
// register staging), into a four-stage ring: the loads of k-step ks+3 are
// issued during the first half of k-step ks, between its matrix instructions,
// so each has two k-steps to arrive.  The
// wavefronts read their fragments one half k-step ahead (the second half of
// ks while multiplying the first, the first half of ks+1 while multiplying the
// second), and decode each 8-element chunk while the previous chunk's matrix
// instructions run.  One barrier per k-step.  Each operand byte is fetched
// once per workgroup.
//
// LDS stage layout (bytes), "lane" = l32 + 32*h of the consuming wavefront,
// RB = 2*TM row blocks and CB = 2*TN column blocks of 32:
//   A codes  [row block RB][half p 2][lane 64][16]  rows rb*32+l32, bytes h*32+p*16 of the k-step
//   B codes  [col block CB][half p 2][lane 64][16]  packed unit kg = 2h+p of column cb*32+l32
//   A scales [row block RB][lane 64][4]             block scales 4h..4h+3 of the row
//   B scales [col block CB][lane 64][4]
// so every fragment read is one ds_read_b128 (or b32) of a contiguous,
// bank-conflict-free 1 KB (256 B) span.  256 x 256 tiles hold their scales as
//   A scales [row 256][16]   the row's scale bytes of the aligned k-step pair
//   B scales [column 256][8]
// instead (one 16-byte load per wavefront and operand; the 4-byte scale reads
// then see 2- to 4-way bank conflicts, a few cycles per k-step).
//
// Workgroups are numbered so that the ones sharing an XCD (consecutive
// hardware ids go round-robin over the 8 XCDs) work on a compact group of
// tiles and reuse operands from that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kGroupM = 8;   // tile rows per group of the grouped tile order

template <int TM, int TN>
struct TileGeom {
    static constexpr int BM = 2 * TM * 32, BN = 2 * TN * 32;
    static constexpr int RB = BM / 32, CB = BN / 32;               // 32-row / 32-column blocks
    static constexpr int A_CODES = RB * 2 * 1024;
    static constexpr int B_CODES = CB * 2 * 1024;
    // 256 x 256 tiles (K a multiple of 256) load their block scales with 16-byte
    // loads, one per wavefront: A as [row 256][16 B] (the row's scale bytes of an
    // aligned pair of k-steps), B as [column 256][8 B] (waves 0 and 1, 128
    // columns each; waves 2 and 3 load into a spare 1 KB): 10 loads per wavefront
    // and k-step instead of 12 (A/B on one MI355X: large prefill product 11.99 ->
    // 11.95 ms, nGPT 208.4 -> 207.2 us).  Smaller tiles keep 4-byte scale loads: slabs of 256 B as
    // [block][lane 64][4 B], with fewer than four row or column blocks some
    // wavefronts loading into a spare slab.
    static constexpr bool WIDE = (RB == 8 && CB == 8);
    static constexpr int A_SC = WIDE ? RB * 32 * 16 : RB * 256;
    static constexpr int B_SC = WIDE ? CB * 32 * 8 : CB * 256;
    static constexpr int SPARE = WIDE ? 1024 : (RB % 4 != 0 || CB % 4 != 0) ? 256 : 0;
    static constexpr int STAGE = A_CODES + B_CODES + A_SC + B_SC + SPARE;
    static constexpr int A_CHUNKS = A_CODES / 16 / 256, B_CHUNKS = B_CODES / 16 / 256;   // per thread
    static constexpr int AS_WORDS = WIDE ? 1 : (RB + 3) / 4, BS_WORDS = WIDE ? 1 : (CB + 3) / 4;
    static_assert(!WIDE || 4 * STAGE <= 160 * 1024, "four stages fit the LDS");
    static_assert(A_CHUNKS * 16 * 256 == A_CODES && B_CHUNKS * 16 * 256 == B_CODES, "whole code slabs per wave");
};

struct TileSrc {
    rsrc_t ac, as, bc, bs;
    uint32_t a_lane, as_lane, b_lane, bs_lane;   // per-lane offsets inside a 32-row / 32-column block
    uint32_t as16_lane, bs16_lane;               // the same for the 16-byte scale loads (64 rows / 128 columns)
    uint32_t a_tile, as_tile, b_tile, bs_tile;   // offsets of the workgroup tile's first block
    uint32_t a_blk, as_blk, b_blk, bs_blk;       // advance per 32-row / 32-column block
};

// One buffer load that writes LDS directly: lane l's 16 (or 4) bytes land at
// lds + 16*l (4*l).  lds must be the same for the whole wavefront.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, (int)voff, (int)soff, 0, 0);
}

// A scalar offset past the end of every buffer: the load touches no memory and
// writes zeros, so steps beyond the last k-step keep the load count per step
// constant (the vmcnt bookkeeping below relies on it) at no memory cost.
constexpr uint32_t kDeadOffset = 0x80000000u;

// Global -> LDS stage for k-step ks, one load at a time: load idx (0 ..
// kLoads-1) of wavefront w moves slab w + 4*u of the A codes, B codes, A
// scales or B scales (a slab is 1 KB of codes or 256 B of scales).
template <int TM, int TN>
struct DmaPlan {
    using G = TileGeom<TM, TN>;
    static constexpr int kLoads = G::A_CHUNKS + G::B_CHUNKS + G::AS_WORDS + G::BS_WORDS;
};
template <int TM, int TN>
__device__ __forceinline__ void dma_one(uint8_t* stage, const TileSrc& s, uint32_t ks, bool live, int wave, int idx) {
    using G = TileGeom<TM, TN>;
    if (idx < G::A_CHUNKS) {
        const int slab = wave + 4 * idx, rb = slab >> 1, p = slab & 1;
        dma16(s.ac, stage + slab * 1024, s.a_lane, live ? s.a_tile + rb * s.a_blk + ks * 64 + p * 16 : kDeadOffset);
        return;
    }
    idx -= G::A_CHUNKS;
    if (idx < G::B_CHUNKS) {
        const int slab = wave + 4 * idx, cb = slab >> 1, p = slab & 1;
        dma16(s.bc, stage + G::A_CODES + slab * 1024, s.b_lane,
              live ? s.b_tile + cb * s.b_blk + ks * 1024 + p * 256 : kDeadOffset);
        return;
    }
    idx -= G::B_CHUNKS;
    uint8_t* const spare = stage + G::A_CODES + G::B_CODES + G::A_SC + G::B_SC;
    if constexpr (G::WIDE) {
        if (idx == 0) {   // A scales of tile rows 64*wave .. +63, the k-step pair holding ks
            dma16(s.as, stage + G::A_CODES + G::B_CODES + wave * 1024, s.as16_lane,
                  live ? s.as_tile + 2 * (uint32_t)wave * s.as_blk + (ks & ~1u) * 8 : kDeadOffset);
            return;
        }
        const bool own = wave < 2;   // B scales of tile columns 128*wave .. +127
        dma16(s.bs, own ? stage + G::A_CODES + G::B_CODES + G::A_SC + wave * 1024 : spare, s.bs16_lane,
              live && own ? s.bs_tile + 4 * (uint32_t)wave * s.bs_blk + ks * 128 : kDeadOffset);
        return;
    }
    if (idx < G::AS_WORDS) {
        const int slab = wave + 4 * idx;
        const bool own = slab < G::RB;   // (wave-uniform)
        dma4(s.as, own ? stage + G::A_CODES + G::B_CODES + slab * 256 : spare, s.as_lane,
             live && own ? s.as_tile + slab * s.as_blk + ks * 8 : kDeadOffset);
        return;
    }
    idx -= G::AS_WORDS;
    const int slab = wave + 4 * idx;
    const bool own = slab < G::CB;
    dma4(s.bs, own ? stage + G::A_CODES + G::B_CODES + G::A_SC + slab * 256 : spare, s.bs_lane,
         live && own ? s.bs_tile + slab * s.bs_blk + ks * 128 : kDeadOffset);
}
template <int TM, int TN>
__device__ __forceinline__ void stage_dma(uint8_t* stage, const TileSrc& s, uint32_t ks, bool live, int wave) {
#pragma unroll
    for (int idx = 0; idx < DmaPlan<TM, TN>::kLoads; ++idx) dma_one<TM, TN>(stage, s, ks, live, wave, idx);
}

// Wait until at most n of this wavefront's buffer loads are outstanding
// (they complete in issue order); the other counters are left alone.
template <int n>
__device__ __forceinline__ void wait_vmem() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Raw fragments of one wavefront for half p of a k-step, and the block scales
// of a whole k-step, read from an LDS stage.
template <int TM, int TN>
struct Frags {
    uint4 a[TM], b[TN];
};
template <int TM, int TN>
__device__ __forceinline__ void read_half(Frags<TM, TN>& f, const uint8_t* stage, int p, int wm, int wn, int lane) {
    using G = TileGeom<TM, TN>;
#pragma unroll
    for (int i = 0; i < TM; ++i)
        f.a[i] = *reinterpret_cast<const uint4*>(stage + ((wm * TM + i) * 2 + p) * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j)
        f.b[j] = *reinterpret_cast<const uint4*>(stage + G::A_CODES + ((wn * TN + j) * 2 + p) * 1024 + lane * 16);
}
template <int TM, int TN>
struct RawScales {
    uint32_t a[TM], b[TN];
};
template <int TM, int TN>
__device__ __forceinline__ void read_raw_scales(RawScales<TM, TN>& sc, const uint8_t* stage, int wm, int wn, int lane,
                                                int odd) {
    using G = TileGeom<TM, TN>;
    const uint8_t* const as = stage + G::A_CODES + G::B_CODES;
    const uint8_t* const bs = as + G::A_SC;
    if constexpr (G::WIDE) {
        const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            sc.a[i] = *reinterpret_cast<const uint32_t*>(as + ((wm * TM + i) * 32 + l32) * 16 + odd * 8 + h * 4);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            sc.b[j] = *reinterpret_cast<const uint32_t*>(bs + ((wn * TN + j) * 32 + l32) * 8 + h * 4);
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            sc.a[i] = *reinterpret_cast<const uint32_t*>(as + (wm * TM + i) * 256 + lane * 4);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            sc.b[j] = *reinterpret_cast<const uint32_t*>(bs + (wn * TN + j) * 256 + lane * 4);
    }
}

// Block scales of one k-step as FP16 pairs.  The 7 magnitude bits of an E4M3
// byte placed at FP16 bits 13..7 give S * 2^-8 exactly (an FP16 subnormal for
// the E4M3 subnormals).  lo holds bytes 0 and 2 of a lane's scale word, hi
// bytes 1 and 3, so 16-element block i (0..3) has its scale in half i >> 1 of
// (i & 1 ? hi : lo).
struct ScalePair {
    uint32_t lo, hi;
};
__device__ __forceinline__ ScalePair split_scales(uint32_t w) {
    return {(w << 7) & 0x3F803F80u, (w >> 1) & 0x3F803F80u};
}
__device__ __forceinline__ half2v block_scale(const ScalePair& sp, int i) {
    const half2v pr = __builtin_bit_cast(half2v, (i & 1) ? sp.hi : sp.lo);
    return (i >> 1) ? half2v{pr[1], pr[1]} : half2v{pr[0], pr[0]};
}
template <int TM, int TN>
struct Scales {
    ScalePair a[TM], b[TN];
};
template <int TM, int TN>
__device__ __forceinline__ void split_all(Scales<TM, TN>& out, const RawScales<TM, TN>& in) {
#pragma unroll
    for (int i = 0; i < TM; ++i) out.a[i] = split_scales(in.a[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) out.b[j] = split_scales(in.b[j]);
}

// Two elements of a chunk: the conversion's power-of-two scale makes each code
// exactly code * 256, and the packed multiply by S * 2^-8 gives code * S
// exactly (at most 6 significant bits, inside [2^-10, 2688]).
template <int BYTE>
__device__ __forceinline__ half2v dec2(uint32_t w, half2v s2) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, BYTE) * s2;
}

// Decoded operands of one 8-element chunk c of half p.
template <int TM, int TN>
struct Chunk {
    half8 a[TM], b[TN];
};

// Piece k (0 .. 2*(TM+TN)-1) of decoding chunk c of half p: half (k & 1) of
// operand k >> 1 (A rows first, then B columns).
template <int TM, int TN>
__device__ __forceinline__ void decode_piece(Chunk<TM, TN>& d, const Frags<TM, TN>& f, const Scales<TM, TN>& sc,
                                             int p, int c, int k) {
    const int o = k >> 1, blk = 2 * p + (c >> 1);
    const bool is_a = o < TM;
    const uint32_t w = is_a ? word_of(f.a[o], c) : word_of(f.b[o - TM], c);
    const half2v s2 = block_scale(is_a ? sc.a[o] : sc.b[o - TM], blk);
    half8& v = is_a ? d.a[o] : d.b[o - TM];
    if ((k & 1) == 0) {
        const half2v e0 = dec2<0>(w, s2), e1 = dec2<1>(w, s2);
        v.s0 = e0[0]; v.s1 = e0[1]; v.s2 = e1[0]; v.s3 = e1[1];
    } else {
        const half2v e2 = dec2<2>(w, s2), e3 = dec2<3>(w, s2);
        v.s4 = e2[0]; v.s5 = e2[1]; v.s6 = e3[0]; v.s7 = e3[1];
    }
}
template <int TM, int TN>
__device__ __forceinline__ void decode_chunk(Chunk<TM, TN>& d, const Frags<TM, TN>& f, const Scales<TM, TN>& sc, int p,
                                             int c) {
#pragma unroll
    for (int k = 0; k < 2 * (TM + TN); ++k) decode_piece<TM, TN>(d, f, sc, p, c, k);
}

// One k-step held in stage `cur`, as 8 chunks (p = q >> 2, c = q & 3).  On
// entry f[0] holds half 0 of this k-step, sc its scales and d[0] its chunk 0
// decoded; on exit the same holds for the next k-step, read from `nxt`.
//
// The instruction order is fixed by hand (the scheduler may not move anything
// across the fences): each matrix instruction of chunk q is followed by an
// equal share of the decode of chunk q+1, so the vector ALU work runs while
// the matrix core is busy; the loads of k-step t+3 into dma_stage ride on the
// matrix instructions of the k-step the same way, one every few instructions.  LDS reads are issued a whole half k-step before
// their data is decoded; the scales of the next k-step are split during
// chunk 5.
template <int TM, int TN>
__device__ __forceinline__ void kstep(float16v (&acc)[TM][TN], Frags<TM, TN> (&f)[2], Scales<TM, TN>& sc,
                                      Chunk<TM, TN> (&d)[2], const uint8_t* cur, const uint8_t* nxt, int wm, int wn,
                                      int lane, uint8_t* dma_stage, const TileSrc& src, uint32_t dma_ks, bool dma_live,
                                      int wave, int nxt_odd) {
    constexpr int kMma = TM * TN, kPieces = 2 * (TM + TN), kOps = TM + TN;
    constexpr int kLoads = DmaPlan<TM, TN>::kLoads;
    // one load after every kDmaSpacing-th matrix instruction (as far as the k-step's instructions reach):
    // spread over the first half of a 256 x 256 k-step rather than back to back, the loads of the four
    // wavefronts queue less at the texture unit (random operands, 16384^3: 6313 -> 6210 us on MI355X)
    constexpr int kDmaSpacing = (8 * kMma) / kLoads >= 8 ? 4 : (8 * kMma) / kLoads >= 2 ? 2 : 1;
    static_assert(kLoads <= (8 * kMma + kDmaSpacing - 1) / kDmaSpacing, "every load of the k-step is issued");
    static_assert(kPieces % kMma == 0 || kMma % kPieces == 0, "pieces must spread evenly");
    RawScales<TM, TN> raw;
    Scales<TM, TN> nsc;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (q == 0) read_half<TM, TN>(f[1], cur, 1, wm, wn, lane);
        if (q == 4) {
            read_half<TM, TN>(f[0], nxt, 0, wm, wn, lane);
            read_raw_scales<TM, TN>(raw, nxt, wm, wn, lane, nxt_odd);
        }
        __builtin_amdgcn_sched_barrier(0);
        // next chunk: (q+1) of this k-step, or chunk 0 of the next one
        const int np = q < 7 ? (q + 1) >> 2 : 0, nc = q < 7 ? (q + 1) & 3 : 0;
        Chunk<TM, TN>& nd = d[(q + 1) & 1];
        const Frags<TM, TN>& nf = f[np];
#pragma unroll
        for (int m = 0; m < kMma; ++m) {
            const int i = m / TN, j = m % TN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d[q & 1].a[i], d[q & 1].b[j], acc[i][j], 0, 0, 0);
            if ((q * kMma + m) % kDmaSpacing == 0 && (q * kMma + m) / kDmaSpacing < kLoads)
                dma_one<TM, TN>(dma_stage, src, dma_ks, dma_live, wave, (q * kMma + m) / kDmaSpacing);
            if (q == 5) {
#pragma unroll
                for (int o = m; o < kOps; o += kMma) {
                    if (o < TM) nsc.a[o] = split_scales(raw.a[o]);
                    else nsc.b[o - TM] = split_scales(raw.b[o - TM]);
                }
            }
#pragma unroll
            for (int k = m * kPieces / kMma; k < (m + 1) * kPieces / kMma; ++k)
                decode_piece<TM, TN>(nd, nf, q < 7 ? sc : nsc, np, nc, k);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    sc = nsc;
}

// ---------------------------------------------------------------------------
// Work split: one workgroup per output tile, 256 x 256 (one workgroup per
// compute unit: 147 KB of LDS, all 512 registers of each SIMD), 128 x 128
// (two per compute unit) or 64 x 64 (four per compute unit).  The host picks
// the shape that finishes first, counting rounds of workgroups over the
// compute units: small products get the small tiles, so that more compute
// units have work.  Every output element sums its k-steps in the same order
// with any shape, so the choice never changes a result.
// ---------------------------------------------------------------------------
// logical workgroup id: the workgroups of one XCD (hardware ids go round-robin
// over the XCDs) get consecutive logical ids
__device__ __forceinline__ int xcd_order(int hw, int n) {
    const int per_xcd = (n + kXcds - 1) / kXcds;
    const int full = n - (per_xcd - 1) * kXcds;   // XCDs that get per_xcd workgroups
    const int xcd = hw % kXcds, slot = hw / kXcds;
    return (xcd < full ? xcd * per_xcd : full * per_xcd + (xcd - full) * (per_xcd - 1)) + slot;
}

// Tile lid in grouped order: kGroupM tile rows at a time, column-major inside the group.
__device__ __forceinline__ void tile_coords(int lid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int group = lid / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = lid - group * kGroupM * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// Per-lane and per-block source offsets (the per-tile ones are set by point_at).
template <int TM, int TN>
__device__ __forceinline__ TileSrc make_src(int64_t M, int64_t K, int64_t n_pad, const uint8_t* a_codes,
                                            const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                            int lane) {
    const int l32 = lane & 31, h = lane >> 5;
    const uint32_t KS = (uint32_t)(K / kPackK);
    TileSrc s;
    s.ac = make_rsrc(a_codes, (uint64_t)M * K / 2);        // rows >= M read as zero
    s.as = make_rsrc(a_scales, (uint64_t)M * K / 16);
    s.bc = make_rsrc(w_codes, (uint64_t)n_pad * K / 2);
    s.bs = make_rsrc(w_scales, (uint64_t)n_pad * K / 16);
    s.a_lane = (uint32_t)l32 * (uint32_t)(K / 2) + h * 32;
    s.as_lane = (uint32_t)l32 * (uint32_t)(K / 16) + h * 4;
    s.b_lane = (uint32_t)(l32 >> 4) * KS * 1024 + (2 * h) * 256 + (l32 & 15) * 16;
    s.bs_lane = (uint32_t)(l32 >> 4) * KS * 128 + (l32 & 15) * 8 + h * 4;
    s.as16_lane = (uint32_t)lane * (uint32_t)(K / 16);                     // row `lane` of a 64-row group
    s.bs16_lane = (uint32_t)(lane >> 3) * KS * 128 + (lane & 7) * 16;      // rows 2(lane%8), +1 of packed block lane/8
    s.a_blk = 32 * (uint32_t)(K / 2);
    s.as_blk = 32 * (uint32_t)(K / 16);
    s.b_blk = 2 * KS * 1024;     // 32 columns = two 16-row packed blocks
    s.bs_blk = 2 * KS * 128;
    return s;
}
// Source offsets of tile (tm, tn) starting at k-step k0.
template <int TM, int TN>
__device__ __forceinline__ void point_at(TileSrc& s, int tm, int tn, uint32_t k0) {
    using G = TileGeom<TM, TN>;
    s.a_tile = (uint32_t)tm * G::RB * s.a_blk + k0 * 64;
    s.as_tile = (uint32_t)tm * G::RB * s.as_blk + k0 * 8;
    s.b_tile = (uint32_t)tn * G::CB * s.b_blk + k0 * 1024;
    s.bs_tile = (uint32_t)tn * G::CB * s.bs_blk + k0 * 128;
}

// Multiply one tile over nsteps k-steps (the source offsets already point at
// the first one) into acc.  On return no load is in flight and every
// wavefront is past its last LDS read.
template <int TM, int TN>
__device__ __forceinline__ void tile_product(float16v (&acc)[TM][TN], uint8_t* const (&stg)[4], const TileSrc& s,
                                             uint32_t nsteps, int wave, int wm, int wn, int lane) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Ring invariant at the top of k-step t: k-steps up to t+1 are in LDS and
    // visible to every wavefront, k-step t+2 is in flight.
    constexpr int kLoadsPerStep = DmaPlan<TM, TN>::kLoads;
    stage_dma<TM, TN>(stg[0], s, 0, true, wave);
    stage_dma<TM, TN>(stg[1], s, 1, nsteps > 1, wave);
    stage_dma<TM, TN>(stg[2], s, 2, nsteps > 2, wave);
    wait_vmem<kLoadsPerStep>();
    __builtin_amdgcn_s_barrier();

    Frags<TM, TN> f[2];
    Chunk<TM, TN> d[2];
    Scales<TM, TN> sc;
    {
        RawScales<TM, TN> raw;
        read_half<TM, TN>(f[0], stg[0], 0, wm, wn, lane);
        read_raw_scales<TM, TN>(raw, stg[0], wm, wn, lane, 0);
        split_all<TM, TN>(sc, raw);
    }
    decode_chunk<TM, TN>(d[0], f[0], sc, 0, 0);
    // The k-step count is rounded up to a multiple of 4 so the loop body has no
    // branches (the compiler's per-stage wait tracking does not survive them);
    // the extra k-steps load zeros (scale 0) and add nothing.
    const uint32_t n4 = (nsteps + 3) & ~3u;
    for (uint32_t t0 = 0; t0 < n4; t0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t t = t0 + u;
            // stage (t+3)%4 was last read during k-step t-1, before the last barrier;
            // kstep issues the loads of k-step t+3 into it
            kstep<TM, TN>(acc, f, sc, d, stg[u], stg[(u + 1) & 3], wm, wn, lane, stg[(u + 3) & 3], s, t + 3,
                          t + 3 < nsteps, wave, (u + 1) & 1);
            wait_vmem<kLoadsPerStep>();   // k-step t+2 has landed; t+3 may still be in flight
            __builtin_amdgcn_s_barrier();
        }
    }
    wait_vmem<0>();   // the zero loads past the end, before the stages are reused
}

template <int TM, int TN, bool GATED, bool BF16>
__device__ __forceinline__ void store_tile_cols(const float16v (&acc)[TM][TN], int tm, int tn, int64_t M, int64_t N,
                                                const float* __restrict__ g_x, const float* __restrict__ colscale,
                                                float* __restrict__ y, int64_t ld_y, const Epilogue& gp, int wm,
                                                int wn, int lane) {
    using G = TileGeom<TM, TN>;
    const int l32 = lane & 31, h = lane >> 5;
    const float gx = g_x[0];
    const int64_t n0 = (int64_t)tn * G::BN + wn * (TN * 32) + l32;
    // per column block: its scale (and gate parameters); the stores then walk the rows with the column
    // blocks innermost, so the pieces of one output row's line are written back to back
    float cs[TN];
    GateCol gc[TN];
    bool live[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + j * 32;
        live[j] = n < N;
        cs[j] = live[j] ? gx * colscale[n] : 0.0f;
        gc[j] = GateCol{0, 0.0f, 0.0f};
        if constexpr (GATED) {
            if (live[j]) gc[j] = gate_col(n, gp);
        }
    }
    const int64_t m0 = (int64_t)tm * G::BM + wm * (TM * 32) + h * 4;
    using Out = std::conditional_t<BF16, uint16_t, float>;
    if ((int64_t)(tm + 1) * G::BM <= M && (int64_t)(tn + 1) * G::BN <= N) {
        // Interior tile: no bounds to check.  One lane pointer; each row adds a
        // uniform multiple of ld_y and the column blocks are immediate offsets.
        // (rows 0..3, 8..11, 16..19, 24..27 of each 32-row block: the pointer steps one row, or five
        // after every fourth)
        Out* pr = reinterpret_cast<Out*>(y) + m0 * ld_y + n0;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float v = acc[i][j][r] * cs[j];
                    if constexpr (GATED) v = gate_apply(v, gc[j]);
                    if constexpr (BF16) pr[j * 32] = f32_to_bf16_rne(v);
                    else pr[j * 32] = v;
                }
                pr += (r & 3) == 3 ? 5 * ld_y : ld_y;
            }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + i * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if (!live[j]) continue;
                    float v = acc[i][j][r] * cs[j];
                    if constexpr (GATED) v = gate_apply(v, gc[j]);
                    if constexpr (BF16) reinterpret_cast<Out*>(y)[m * ld_y + n0 + j * 32] = f32_to_bf16_rne(v);
                    else reinterpret_cast<Out*>(y)[m * ld_y + n0 + j * 32] = v;
                }
            }
        }
    }
}

// Y = acc * g_x * colscale for one tile (rows >= M and columns >= N skipped).
// EPI bit 0: gates, evaluated only in the tiles that hold gate columns;
// EPI bit 1: bf16 output.  Each combination is its own kernel, so the store
// loops stay straight-line code over the accumulator registers and the plain
// kernel carries nothing of the others.
constexpr int kEpiGates = 1, kEpiBf16 = 2;

template <int TM, int TN, int EPI>
__device__ __forceinline__ void store_tile(const float16v (&acc)[TM][TN], int tm, int tn, int64_t M, int64_t N,
                                           const float* __restrict__ g_x, const float* __restrict__ colscale,
                                           float* __restrict__ y, int64_t ld_y, const Epilogue& gp, int wm, int wn,
                                           int lane) {
    using G = TileGeom<TM, TN>;
    constexpr bool BF16 = (EPI & kEpiBf16) != 0;
    if constexpr ((EPI & kEpiGates) != 0) {
        if (gates_touch((int64_t)tn * G::BN, (int64_t)(tn + 1) * G::BN, gp)) {
            store_tile_cols<TM, TN, true, BF16>(acc, tm, tn, M, N, g_x, colscale, y, ld_y, gp, wm, wn, lane);
            return;
        }
    }
    store_tile_cols<TM, TN, false, BF16>(acc, tm, tn, M, N, g_x, colscale, y, ld_y, gp, wm, wn, lane);
}

#define NVFP4_TILE_KERNEL_ARGS                                                                                   \
    int64_t M, const uint8_t *__restrict__ a_codes, const uint8_t *__restrict__ a_scales,                        \
        const float *__restrict__ g_x, const uint8_t *__restrict__ w_codes, const uint8_t *__restrict__ w_scales, \
        const float *__restrict__ colscale, int64_t N, int64_t n_pad, int64_t K, float *__restrict__ y,           \
        int64_t ld_y

// One whole tile per workgroup.
template <int TM, int TN, int EPI>
__global__ __launch_bounds__(256) void gemm_tile_kernel(NVFP4_TILE_KERNEL_ARGS, Epilogue gp, int tiles_m,
                                                        int tiles_n) {
    using G = TileGeom<TM, TN>;
    // Four separate arrays rather than one: the compiler then tells the stages
    // apart and waits only for the loads that target the stage being read.
    __shared__ __attribute__((aligned(16))) uint8_t st0[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3[G::STAGE];
    uint8_t* const stg[4] = {st0, st1, st2, st3};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_coords(xcd_order(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
    TileSrc s = make_src<TM, TN>(M, K, n_pad, a_codes, a_scales, w_codes, w_scales, lane);
    point_at<TM, TN>(s, tm, tn, 0);
    float16v acc[TM][TN];
    tile_product<TM, TN>(acc, stg, s, (uint32_t)(K / kPackK), wave, wm, wn, lane);
    store_tile<TM, TN, EPI>(acc, tm, tn, M, N, g_x, colscale, y, ld_y, gp, wm, wn, lane);
}

// Host side.  Time per round of workgroups, relative: a round of 128 x 128
// tiles (two per compute unit) takes about 0.53 of a round of 256 x 256 tiles
// (measured on MI355X over K = 4096; the ratio barely moves with K).
constexpr int kTileRoundsSmall = 53, kTileRoundsLarge = 100;

// Time of a launch in those units: whole rounds of 256x256 tiles (one per
// compute unit) or of 128x128 tiles (two per compute unit).
static int64_t cost_large(int64_t M, int64_t cols_pad) {
    const int64_t tiles = ((M + 255) / 256) * (cols_pad / 256);
    return (tiles + kComputeUnits - 1) / kComputeUnits * kTileRoundsLarge;
}
static int64_t cost_small(int64_t M, int64_t cols_pad) {
    const int64_t tiles = ((M + 127) / 128) * (cols_pad / 128);
    return (tiles + 2 * kComputeUnits - 1) / (2 * kComputeUnits) * kTileRoundsSmall;
}

// Columns [0, split) on 256x256 tiles and [split, n_padded) on 128x128 tiles:
// split = n_padded (all large), 0 (all small), or the last multiple of 256 at
// or below n when a ragged column edge (e.g. the 96 gate columns past 16384 of
// a fused GDN projection) would otherwise cost a whole extra round of large
// tiles.  Every output element is the same sum whichever tile computes it.
static int64_t column_split(int64_t M, const nvfp4_weight_desc& d) {
    if (M <= 128) return 0;
    if (d.k % 256 != 0) return 0;   // 256 x 256 tiles read their A scales by aligned pairs of k-steps
    const int64_t all_large = cost_large(M, d.n_padded), all_small = cost_small(M, d.n_padded);
    const int64_t edge = d.n / 256 * 256;
    const int64_t mixed = (edge > 0 && edge < d.n_padded) ? cost_large(M, edge) + cost_small(M, d.n_padded - edge)
                                                           : INT64_MAX;
    if (mixed < all_large && mixed < all_small) return edge;
    return all_small < all_large ? 0 : d.n_padded;
}

size_t gemm_workspace_bytes(int64_t, const nvfp4_weight_desc&) { return 0; }

// One launch over the weight's columns [c0, c1) (multiples of the tile width;
// c1 <= n_padded): operand, column-scale and output pointers move to column
// c0, the gate columns shift with them.
template <int TM, int TN>
static hipError_t launch_tiles(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                               const nvfp4_weight_desc& d, int64_t c0, int64_t c1, float* y, int64_t ld_y,
                               const Epilogue& gp_all, hipStream_t stream) {
    constexpr int BM = 64 * TM, BN = 64 * TN;
    const uint8_t* blob = static_cast<const uint8_t*>(d.blob);
    const uint8_t* wc = blob + d.codes_offset + c0 * d.k / 2;
    const uint8_t* wsc = blob + d.scales_offset + c0 * d.k / 16;
    const float* cs = reinterpret_cast<const float*>(blob + d.colscale_offset) + c0;
    float* yc = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(y) + c0 * (gp_all.out_bf16 ? 2 : 4));
    const int64_t n = (d.n < c1 ? d.n : c1) - c0, n_pad = c1 - c0;
    Epilogue gp = gp_all;
    gp.a_col -= (int32_t)c0;
    gp.b_col -= (int32_t)c0;
    // gates only where a gate column falls inside this launch
    const bool gated = (gp.n_a > 0 && 0 < gp.a_col + gp.n_a && gp.a_col < n) ||
                       (gp.n_b > 0 && 0 < gp.b_col + gp.n_b && gp.b_col < n);
    // tiles up to the last real column (the padding columns past it are never stored)
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
    const int epi = (gated ? kEpiGates : 0) | (gp.out_bf16 ? kEpiBf16 : 0);
    auto kern = epi == 0 ? gemm_tile_kernel<TM, TN, 0>
              : epi == kEpiGates ? gemm_tile_kernel<TM, TN, kEpiGates>
              : epi == kEpiBf16 ? gemm_tile_kernel<TM, TN, kEpiBf16>
                                : gemm_tile_kernel<TM, TN, kEpiGates | kEpiBf16>;
    hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(256), 0, stream, M, a_codes,
                       a_scales, g_x, wc, wsc, cs, n, n_pad, d.k, yc, ld_y, gp, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_gemm(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                       const nvfp4_weight_desc& d, float* y, int64_t ld_y, void* ws, size_t, const Epilogue& gp,
                       hipStream_t stream) {
    if (skinny_applies(M, d)) {
        return launch_skinny(M, nullptr, NVFP4_IN_BF16, 0, const_cast<float*>(g_x), NVFP4_G_GIVEN,
                             const_cast<uint8_t*>(a_codes), const_cast<uint8_t*>(a_scales), false, d, y, ld_y, ws,
                             gp, stream);
    }
    const int64_t split = column_split(M, d);
    if (split > 0) {
        const hipError_t e = launch_tiles<4, 4>(M, a_codes, a_scales, g_x, d, 0, split, y, ld_y, gp, stream);
        if (e != hipSuccess || split == d.n_padded) return e;
    }
    // 64 x 64 tiles (four times the workgroups, each a quarter of the work) where 128 x 128 tiles would
    // leave units idle: a few hundred tokens, or the ragged column edge of a fused projection after the
    // large tiles.  Taken when the narrow tiles fit one per unit, or when the small ones would leave more
    // than half of the units idle (measured, N = K = 5120: 32-192 tokens 36-38 -> 22-25 us, 256 tokens
    // 38.9 -> 35.1 us, 512 tokens 42.9 -> 51.3 us, so 512 stays on 128 x 128)
    const int64_t rest_cols = (d.n < d.n_padded ? d.n : d.n_padded) - split;
    const int64_t small_tiles = ((M + 127) / 128) * ((rest_cols + 127) / 128);
    const int64_t narrow_tiles = ((M + 63) / 64) * ((rest_cols + 63) / 64);
    if (narrow_tiles <= kComputeUnits || 2 * small_tiles < kComputeUnits)
        return launch_tiles<1, 1>(M, a_codes, a_scales, g_x, d, split, d.n_padded, y, ld_y, gp, stream);
    return launch_tiles<2, 2>(M, a_codes, a_scales, g_x, d, split, d.n_padded, y, ld_y, gp, stream);
}

}  // namespace nvfp4
