// mx_gemm.hip -- grouped MXFP4 GEMM on the CDNA4 block-scaled FP4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E2M1, FP32 accumulation).
//
// Operand layout the MFMA reads (one wave, 32x32 output, K = 64): lane l
// supplies row (l % 32) of its operand and K elements [32 (l / 32), +32) as
// 16 bytes (even element in the low nibble) plus that 32-block's UE8M0 scale
// byte.  A 32-element MX block is exactly one lane's 16-byte operand and one
// scale byte, so the row-major code and scale layouts written by the
// quantizers are consumed as they are.  Accumulator: lane l, register e holds
// D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].
//
// The MFMA's first operand is the weight tile (rows = output columns n) and
// its second the activation tile (rows = output rows m), so D = C^T per
// 32x32 block and each lane ends up holding 4 consecutive output columns of
// one output row: the epilogue stores 8-byte (bf16) or 16-byte (fp32) runs.
//
// Tiling: a workgroup of 8 waves (2 x 4) computes a 256 x 256 tile of one
// group; each wave owns 128 x 64 (8 MFMA blocks, 128 accumulators), two waves
// per SIMD so that one wave's LDS and DMA waits are covered by the other's
// MFMAs (4 waves of 128 x 128, one per SIMD, measured 8-9% slower).  K
// advances 256 per stage, so every operand row contributes one 128-byte
// line per stage (half-line requests cost nearly as much as full
// ones at the L2).  Every operand byte moves global -> LDS by the CDNA
// LDS-DMA loads (global_load_lds_dwordx4 for 16-byte code chunks, 8 lanes per
// row line; global_load_lds_ubyte for scale bytes, each landing as a dword),
// so no staging registers are needed.  The ring has two 80 KiB buffers (all
// of a CU's LDS): stage kt+2 is issued at stage kt's barrier into the buffer
// stage kt has just finished reading, which leaves it a full stage to land.
// The DMA is issued from register-only inline assembly and its completion is
// awaited explicitly (s_waitcnt vmcnt + s_barrier).  A stage runs as four
// K-quarters of 64; operand fragments are double-buffered in registers and
// the next quarter's fragment reads are interleaved one per MFMA with the
// current quarter's MFMAs.
//
// LDS code tiles use an XOR swizzle of the eight 16-byte chunks of a row;
// each row's 8 scale dwords are stored in the order (s0, s2, s4, s6, s1, s3,
// s5, s7), so one 16-byte read gives a lane the scales of its four
// K-quarters.  A chunk at or past the end of the K range is loaded from a
// clamped (valid) address and its scale is forced to 2^-127 on both
// operands, so its products (at most 36 * 2^-254) vanish in the fp32
// accumulation.
//
// Tile order: 32 consecutive tile ids cover 4 M-tiles x 8 N-tiles of one
// group, and blocks of 32 ids are dealt round-robin to the 8 XCDs (work-
// groups are dispatched to XCDs round-robin), so the workgroups resident on
// one XCD share A rows and B columns in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mx.h"
#include "mx_device.h"

using namespace mx;

namespace {

struct GemmArgs {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const int32_t* a_row_index;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const int32_t* off;
    void* c;
    int64_t M, N, K;
    int32_t G;
    int32_t b_scale_2d;
    int32_t group_dim_k;
    int32_t tiles_n;
    int32_t tiles_m;     // group_dim_k = 1: tiles along M per group
    float alpha;
};

constexpr int BM = 256, BN = 256;
constexpr int NW = 8;               // waves per workgroup (two per SIMD)
constexpr int NT = NW * 64;          // threads per workgroup
constexpr int BK = 256;            // K elements per stage: 128 code bytes per row
constexpr int NST = 2;             // LDS ring depth (2 x 80 KiB: all of a CU's LDS)
constexpr int GROUP_M = 4;         // M-tiles per tile-order group
constexpr int XCDS = 8;
constexpr int XCD_BLOCK = 32;      // consecutive tile ids per XCD turn
// one stage in LDS: A codes, B codes (256 rows x 128 bytes each), A and B
// scales (256 rows x 8 dwords each)
constexpr int OFF_A = 0, OFF_B = 32768, OFF_AS = 65536, OFF_BS = 73728;
constexpr int STAGE_BYTES = 81920;
// DMA ops per thread per stage: 16 code moves, 8 A-scale moves, and 8 B-scale
// moves (1D B scales) or 1 (2D B scales: 8 row groups of 32 per tile).
template <bool B2D>
constexpr int dma_per_stage() { return B2D ? 13 : 16; }

// 16-byte chunk swizzle of a 128-byte row: the rows an MFMA operand read
// touches at one chunk index land in distinct 16-byte bank groups whether
// the LDS serves 8 lanes (32 banks: rows r..r+7) or 16 lanes (64 banks: the
// even and the odd rows of r..r+15) of a ds_read_b128 per cycle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// scale dword slot p of a row holds chunk (0, 2, 4, 6, 1, 3, 5, 7)[p], so
// lane half h reads the chunks of its four K-quarters (2 q + h) in one go
__device__ __forceinline__ int sperm(int p) { return p < 4 ? 2 * p : 2 * (p - 4) + 1; }

// LDS-DMA: every lane moves 16 bytes (or 1 byte, zero-extended to a dword)
// from base + voff to LDS byte address lds + 16 lane (or + 4 lane).  M0
// carries the wave's LDS base.  Register operands only; completion is
// awaited with an explicit s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma1(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;   // v_cvt_pk_bf16_f32: round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <bool OUT_BF16, bool B2D>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmArgs p) {
    // 2 x 4 waves of 128 x 64
    constexpr int WM = 128, WN = 64, FM = 4, FN = WN / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    // ---------------- tile id: XCD-aware remap of the workgroup id ----------
    const int64_t wg = blockIdx.x;
    const int64_t xcd = wg % XCDS, j = wg / XCDS;
    int64_t id = (j / XCD_BLOCK) * (XCDS * XCD_BLOCK) + xcd * XCD_BLOCK + (j % XCD_BLOCK);

    // ---------------- tile decode ----------------
    // Groups split M: wave 0 reads all group offsets at once, scans the tile
    // counts ceil(n_g / BM) * tiles_n across its lanes and publishes the
    // group holding tile `id` (one round trip to memory instead of one per
    // group).
    // the tile decode's result lives in the first ring bytes until every
    // thread has read it (the ring fills all 160 KiB of LDS)
    int32_t* tile_group = (int32_t*)lds;
    int g = 0;
    int64_t m_begin = 0, m_end = 0, k_begin = 0, k_end = p.K, mtiles = 0;
    if (p.group_dim_k == 0) {
        if (wave == 0) {
            if (lane == 0) tile_group[0] = -1;
            int64_t running = 0;
            for (int base = 0; base < p.G; base += 64) {
                const int gg = base + lane;
                int64_t t = 0, gb = 0, ge = 0;
                if (gg < p.G) {
                    gb = p.off[gg];
                    ge = p.off[gg + 1];
                    t = (ge - gb + BM - 1) / BM * p.tiles_n;
                }
                int64_t incl = t;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int64_t v = __shfl_up(incl, d);
                    if (lane >= d) incl += v;
                }
                const int64_t start = running + incl - t;
                if (gg < p.G && id >= start && id < start + t) {
                    tile_group[0] = gg;
                    tile_group[1] = (int32_t)(id - start);
                }
                running += __shfl(incl, 63);
            }
        }
        __syncthreads();
        g = __builtin_amdgcn_readfirstlane(tile_group[0]);   // uniform: the DMA takes scalar bases
        if (g < 0) return;                      // past the last tile (uniform)
        id = __builtin_amdgcn_readfirstlane(tile_group[1]);
        __syncthreads();                        // read by all before the ring's first DMA
        m_begin = p.off[g];
        m_end = p.off[g + 1];
        mtiles = (m_end - m_begin + BM - 1) / BM;
    } else {
        const int64_t per = (int64_t)p.tiles_m * p.tiles_n;
        g = (int)(id / per);
        if (g >= p.G) return;
        id -= (int64_t)g * per;
        mtiles = p.tiles_m;
        m_begin = 0;
        m_end = p.M;
        k_begin = p.off[g];
        k_end = p.off[g + 1];
    }
    // grouped order inside the group: GROUP_M M-tiles x all N-tiles, m fastest
    const int64_t span = (int64_t)GROUP_M * p.tiles_n;
    const int64_t sgrp = id / span;
    const int64_t rem = id - sgrp * span;
    const int64_t gm = min((int64_t)GROUP_M, mtiles - sgrp * GROUP_M);
    const int64_t nt = rem / gm;
    const int64_t mt = sgrp * GROUP_M + (rem - nt * gm);
    const int64_t grp_end = m_end;
    m_begin = m_begin + mt * BM;
    m_end = min(grp_end, m_begin + BM);
    const int64_t n_begin = nt * BN;

    const int64_t KB = p.K / 2;      // code bytes per operand row
    const int64_t KS = p.K / 32;     // scale bytes per operand row

    const uint8_t* bcodes = p.b_codes;
    const uint8_t* bscales = p.b_scales;
    if (p.group_dim_k == 0) {
        bcodes += (int64_t)g * p.N * KB;
        bscales += (int64_t)g * (B2D ? (p.N / 32) * KS : p.N * KS);
    }

    // ---------------- per-thread DMA assignments ----------------
    // Code DMA j of thread t fills 16-byte slot t + 256 j of an operand tile:
    // row r = t/8 + 32 j, slot position pc = t % 8 of the row's 128 bytes, so
    // 8 lanes move one full 128-byte line.  Scale DMA j fills dword slot
    // t + 256 j: the same row, scale position pc.
    const int pc = tid & 7;
    const int a_chunk = pc ^ swz(tid >> 3);    // swz(t/8 + 32 j) is the same for every j
    const int s_chunk = sperm(pc);
    constexpr int NJ = 2048 / NT;               // code (and scale) moves per operand per thread
    uint32_t a_off[NJ], b_off[NJ], as_off[NJ], bs_off[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
        const int r = (tid >> 3) + (NT / 8) * jj;
        int64_t m = m_begin + r;
        if (m >= m_end) m = m_end - 1;        // rows past the tile end are never stored
        const int64_t arow = p.a_row_index ? (int64_t)p.a_row_index[m] : m;
        a_off[jj] = (uint32_t)(arow * KB);
        as_off[jj] = (uint32_t)(arow * KS);
        int64_t n = n_begin + r;
        if (n >= p.N) n = p.N - 1;
        b_off[jj] = (uint32_t)(n * KB);
        bs_off[jj] = (uint32_t)(n * KS);
    }
    // 2D B scales: lane l of every wave fetches row group l / 8 of the tile at
    // scale position l % 8, into its wave's own 256-byte copy
    uint32_t bs2_off = 0;
    if (B2D) {
        int64_t grp = n_begin / 32 + (lane >> 3);
        if (grp > p.N / 32 - 1) grp = p.N / 32 - 1;    // groups past N are never stored
        bs2_off = (uint32_t)(grp * KS);
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    const int64_t klen = k_end - k_begin;
    const int nkt = (int)((klen + BK - 1) / BK);
    const int64_t kc0 = k_begin / 32;        // first K-chunk of the range
    const int64_t kc_end = k_end / 32;
    // K chunks relative to kc0 (32-bit: the host bounds an operand row to 4 GiB)
    const int kc_last = (int)(kc_end - kc0) - 1;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
        a_off[jj] += (uint32_t)(kc0 * 16);
        b_off[jj] += (uint32_t)(kc0 * 16);
        as_off[jj] += (uint32_t)kc0;
        bs_off[jj] += (uint32_t)kc0;
    }
    bs2_off += (uint32_t)kc0;

    // stage kt -> LDS buffer `buf`; chunks past the end are clamped in range
    auto issue = [&](int kt, int buf) {
        const uint32_t sb = lds_base + (uint32_t)buf * STAGE_BYTES;
        const int kc = min(kt * 8 + a_chunk, kc_last);
        const int ks = min(kt * 8 + s_chunk, kc_last);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            dma16(p.a_codes, a_off[jj] + (uint32_t)(kc * 16), sb + OFF_A + jj * NT * 16 + wave * 1024);
            dma16(bcodes, b_off[jj] + (uint32_t)(kc * 16), sb + OFF_B + jj * NT * 16 + wave * 1024);
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            dma1(p.a_scales, as_off[jj] + (uint32_t)ks, sb + OFF_AS + jj * NT * 4 + wave * 256);
            if (!B2D) dma1(bscales, bs_off[jj] + (uint32_t)ks, sb + OFF_BS + jj * NT * 4 + wave * 256);
        }
        if (B2D) dma1(bscales, bs2_off + (uint32_t)ks, sb + OFF_BS + wave * 256);
    };

    v16f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int jj = 0; jj < FM; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.0f;

    const int lr = lane & 31;      // operand row within a 32-row MFMA block
    const int lh = lane >> 5;      // which 32-element half of a K-quarter (64)
    // operand rows w*128 + i*32 + lr share swz(lr) for every i, so a fragment
    // read is one per-lane base plus an immediate i * 4096
    const int sw = swz(lr);
    const uint32_t fb_b = OFF_B + (uint32_t)(wn * WN + lr) * 128;
    const uint32_t fb_a = OFF_A + (uint32_t)(wm * WM + lr) * 128;

    struct Frag { v8i b[FN]; v8i a[FM]; };
    struct Scl { uint4 b[FN]; uint4 a[FM]; };   // component q: K-quarter q
    auto read_frag = [&](Frag& f, int buf, int q) {
        const uint8_t* sb = lds + buf * STAGE_BYTES + (((2 * q + lh) ^ sw) * 16);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const uint4 v = *(const uint4*)(sb + fb_b + i * 4096);
            f.b[i] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const uint4 v = *(const uint4*)(sb + fb_a + i * 4096);
            f.a[i] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
    };
    auto read_scl = [&](Scl& s, int buf) {
        const uint8_t* sb = lds + buf * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < FN; ++i)
            s.b[i] = B2D ? *(const uint4*)(sb + OFF_BS + wave * 256 + (wn * FN + i) * 32 + lh * 16)
                         : *(const uint4*)(sb + OFF_BS + (wn * WN + i * 32 + lr) * 32 + lh * 16);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            s.a[i] = *(const uint4*)(sb + OFF_AS + (wm * WM + i * 32 + lr) * 32 + lh * 16);
    };
    auto qsel = [](const uint4& v, int q) { return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w; };
    auto mma = [&](const Frag& f, const Scl& s, int q, bool tail) {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int sb = tail ? 0 : (int)qsel(s.b[i], q);
#pragma unroll
            for (int jj = 0; jj < FM; ++jj) {
                const int sa = tail ? 0 : (int)qsel(s.a[jj], q);
                acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[i], f.a[jj], acc[i][jj], 4, 4, 0, sb, 0, sa);
            }
        }
    };

    // "every DMA but the newest stage's has landed"
    auto wait_all_but_one_stage = [] {
        if (B2D) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    };
    static_assert(dma_per_stage<true>() == 13 && dma_per_stage<false>() == 16, "wait counts");
    // one MFMA block, optionally followed by one piece of the next read
    auto mma1 = [&](const Frag& f, const Scl& s, int q, bool tail, int m) {
        const int i = m / FM, jj = m % FM;
        const int sb = tail ? 0 : (int)qsel(s.b[i], q);
        const int sa = tail ? 0 : (int)qsel(s.a[jj], q);
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[i], f.a[jj], acc[i][jj], 4, 4, 0, sb, 0, sa);
    };
    auto read_piece = [&](Frag& f, int buf, int q, int k) {
        const uint8_t* sb = lds + buf * STAGE_BYTES + (((2 * q + lh) ^ sw) * 16);
        const uint4 v = k < FN ? *(const uint4*)(sb + fb_b + k * 4096) : *(const uint4*)(sb + fb_a + (k - FN) * 4096);
        v8i& d = k < FN ? f.b[k] : f.a[k - FN];
        d = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    };
    auto mma_rd = [&](const Frag& f, const Scl& s, int q, bool tail, Frag& nf, int nbuf, int nq) {
#pragma unroll
        for (int m = 0; m < FN * FM; ++m) {
            mma1(f, s, q, tail, m);
            if (m < FN + FM) read_piece(nf, nbuf, nq, m);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nkt > 0) {
        Frag f0, f1;
        Scl sc, nsc;
        // Stage kt+1's DMA is issued at stage kt-1's barrier, into the buffer
        // stage kt-1 has finished reading; at stage kt's barrier it is the
        // only DMA outstanding, so vmcnt(0) means it has landed.
        issue(0, 0);
        issue(1, 1);
        wait_all_but_one_stage();
        __builtin_amdgcn_s_barrier();
        read_frag(f0, 0, 0);
        read_scl(sc, 0);
        for (int kt = 0; kt < nkt; ++kt) {
            const int buf = kt & 1;
            const int kcl = kt * 8 + lh;              // this lane's chunk in K-quarter 0
            mma_rd(f0, sc, 0, kcl > kc_last, f1, buf, 1);
            mma_rd(f1, sc, 1, kcl + 2 > kc_last, f0, buf, 2);
            mma_rd(f0, sc, 2, kcl + 4 > kc_last, f1, buf, 3);
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            issue(kt + 2, buf);
            read_scl(nsc, buf ^ 1);
            mma_rd(f1, sc, 3, kcl + 6 > kc_last, f0, buf ^ 1, 0);
            sc = nsc;
        }
        // drain the DMA of the two past-the-end stages before the LDS is reused
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // ---------------- epilogue ----------------
    // Each wave stages its 128 x 128 result through LDS one 32-row slab at a
    // time (row pitch padded by 16 bytes against bank conflicts) and stores
    // whole 16-byte runs, so a store instruction covers 4 full row segments
    // of 256 (bf16) or 2 of 512 (fp32) bytes instead of 32 scattered pieces.
    constexpr int EB = OUT_BF16 ? 2 : 4;              // output element bytes
    constexpr int PITCH = WN * EB + 16;                // LDS bytes per staged row
    constexpr int SEGS = WN * EB / 16;                 // 16-byte runs per row
    static_assert(NW * 32 * PITCH <= NST * STAGE_BYTES, "epilogue staging fits the ring");
    __syncthreads();                                   // every wave is done with the ring
    uint8_t* stage_c = lds + wave * 32 * PITCH;
    const int64_t rows_here = m_end - m_begin;
    uint8_t* cbase = (uint8_t*)p.c;
    if (p.group_dim_k == 1) cbase += (int64_t)g * p.M * p.N * EB;
    const float alpha = p.alpha;
    const int64_t col0 = n_begin + wn * WN;            // first output column of this wave
#pragma unroll
    for (int jj = 0; jj < FM; ++jj) {
        // lane (lr, lh) holds row lr of the slab, columns i*32 + 8q + 4lh + (0..3)
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cl = i * 32 + 8 * q + 4 * lh;
                const float v0 = acc[i][jj][4 * q + 0] * alpha;
                const float v1 = acc[i][jj][4 * q + 1] * alpha;
                const float v2 = acc[i][jj][4 * q + 2] * alpha;
                const float v3 = acc[i][jj][4 * q + 3] * alpha;
                uint8_t* dst = stage_c + lr * PITCH + cl * EB;
                if (OUT_BF16)
                    *(uint2*)dst = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                else
                    *(uint4*)dst = make_uint4(__float_as_uint(v0), __float_as_uint(v1),
                                              __float_as_uint(v2), __float_as_uint(v3));
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): the slab is in LDS
        __builtin_amdgcn_wave_barrier();
        const int64_t row_base = m_begin + wm * WM + jj * 32;
#pragma unroll
        for (int k = 0; k < 32 * SEGS / 64; ++k) {
            const int sidx = lane + 64 * k;
            const int r = sidx / SEGS, sg = sidx % SEGS;
            const uint4 v = *(const uint4*)(stage_c + r * PITCH + sg * 16);
            const int64_t col = col0 + sg * (16 / EB);
            if (wm * WM + jj * 32 + r < rows_here && col < p.N)
                *(uint4*)(cbase + ((row_base + r) * p.N + col) * EB) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);            // reads done before the slab is reused
        __builtin_amdgcn_wave_barrier();
    }
}

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

}  // namespace

extern "C" mx_status mx_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* a_row_index,
                                     const uint8_t* b_codes, const uint8_t* b_scales, int b_scale_2d,
                                     const int32_t* group_offsets, int32_t num_groups, int group_dim_k, int64_t M,
                                     int64_t N, int64_t K, float alpha, void* c, mx_dtype ct, mx_stream stream) {
    if (ct != MX_F32 && ct != MX_BF16) return MX_ERR_DTYPE;
    if (M < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_ERR_SHAPE;
    if (num_groups < 1) return MX_ERR_SHAPE;
    if (group_dim_k != 0 && group_dim_k != 1) return MX_ERR_SHAPE;
    if (group_dim_k == 1 && (b_scale_2d || a_row_index)) return MX_ERR_UNSUPPORTED;
    if (!group_offsets) return MX_ERR_NULL;
    if (M == 0) return MX_OK;
    if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return MX_ERR_NULL;
    if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(c)) return MX_ERR_ALIGN;
    // operand rows are addressed by 32-bit byte offsets: each B group and the
    // A rows (wherever a row index can point) must lie within 4 GiB
    if (group_dim_k == 0 && N * (K / 2) > 0xFFFFFFFFLL) return MX_ERR_SHAPE;
    if (group_dim_k == 1 && (M > 0 && (M - 1) * (K / 2) > 0xFFFFFFFFLL || (N - 1) * (K / 2) > 0xFFFFFFFFLL))
        return MX_ERR_SHAPE;

    GemmArgs p;
    p.a_codes = a_codes;
    p.a_scales = a_scales;
    p.a_row_index = a_row_index;
    p.b_codes = b_codes;
    p.b_scales = b_scales;
    p.off = group_offsets;
    p.c = c;
    p.M = M;
    p.N = N;
    p.K = K;
    p.G = num_groups;
    p.b_scale_2d = b_scale_2d ? 1 : 0;
    p.group_dim_k = group_dim_k;
    p.tiles_n = (int32_t)((N + BN - 1) / BN);
    p.tiles_m = (int32_t)((M + BM - 1) / BM);
    p.alpha = alpha;
    int64_t tiles;
    if (group_dim_k == 0)
        tiles = ((M + BM - 1) / BM + num_groups) * p.tiles_n;   // upper bound on sum_g ceil(n_g / BM)
    else
        tiles = (int64_t)num_groups * p.tiles_m * p.tiles_n;
    // the XCD remap is a bijection on multiples of XCDS * XCD_BLOCK
    const int64_t quantum = XCDS * XCD_BLOCK;
    tiles = (tiles + quantum - 1) / quantum * quantum;
    if (tiles > 0x7FFFFFFF) return MX_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (ct == MX_BF16)
        if (b_scale_2d) hipLaunchKernelGGL((gemm_kernel<true, true>), dim3((unsigned)tiles), dim3(NT), 0, s, p);
        else hipLaunchKernelGGL((gemm_kernel<true, false>), dim3((unsigned)tiles), dim3(NT), 0, s, p);
    else
        if (b_scale_2d) hipLaunchKernelGGL((gemm_kernel<false, true>), dim3((unsigned)tiles), dim3(NT), 0, s, p);
        else hipLaunchKernelGGL((gemm_kernel<false, false>), dim3((unsigned)tiles), dim3(NT), 0, s, p);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}
