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
// one output row.
//
// Tiling: a workgroup of 8 waves (2 x 4) computes 256 x 256 tiles; each wave
// owns 128 x 64 (8 MFMA blocks, 128 accumulators), two waves per SIMD so
// that one wave's LDS and DMA waits are covered by the other's MFMAs (4
// waves of 128 x 128, one per SIMD, measured 8-9% slower).  K advances 256
// per stage, so every operand row contributes one 128-byte line per stage
// (half-line requests cost nearly as much as full ones at the L2).  Every
// operand byte moves global -> LDS by the CDNA LDS-DMA loads
// (global_load_lds_dwordx4 for 16-byte code chunks, 8 lanes per row line;
// global_load_lds_ubyte for scale bytes, each landing as a dword), so no
// staging registers are needed.  The ring has two 80 KiB buffers (all of a
// CU's LDS): stage kt+2 is issued at stage kt's barrier into the buffer stage
// kt has just finished reading, which leaves it a full stage to land.  The
// DMA is issued from register-only inline assembly and its completion is
// awaited explicitly (s_waitcnt vmcnt + s_barrier).  A stage runs as four
// K-quarters of 64; each of the quarter's 8 MFMAs is followed by the read of
// the next quarter's fragment piece whose last use it was, into the same
// registers.  A row's four K-quarter scale bytes are packed in one register
// and the MFMA's scale byte-select picks the quarter.
//
// Persistence: one workgroup per CU walks its tiles in snake order (round r
// takes position r P + w, or r P + P - 1 - w on odd rounds), so groups of
// unequal cost (the weight gradient's K follows the routing counts) spread
// evenly.  The ring runs on across tiles: the last two stages of a tile
// issue the next tile's first two, and the last K-quarter already reads its
// first fragments, so a tile starts its MFMAs without a prologue.  The
// epilogue stores straight from the accumulators (two lane-group register
// swaps give 16 rows x 64 contiguous bytes per store) through a buffer
// resource whose range check drops rows and columns outside C, so every wave
// issues a fixed number of stores and the next tile's first barrier leaves
// them in flight.
//
// LDS code tiles use an XOR swizzle of the eight 16-byte chunks of a row.
// K-quarter q of a stage takes chunk 4 h + q in lane half h, so a lane's four
// scale bytes are adjacent in the row: moved one byte per lane, each scale
// lands in a dword of its own (8 per row, one 16-byte read per lane); moved
// in pairs, each pair does (4 per row, one 8-byte read).  Either way the
// rows of an MFMA block sit consecutively, so a block's scale read is one
// contiguous span of LDS, free of bank conflicts.  A chunk at or past the end of the K range is loaded from a
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

#include <type_traits>

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
    int64_t lda, ldb;    // bytes from one code row to the next (A, B)
    int32_t G;
    int32_t b_scale_2d;
    int32_t staged;      // scales in the staged layout (A; with groups along K also B)
    int32_t group_dim_k;
    int32_t tiles_n;
    int32_t tiles_m;     // group_dim_k = 1: tiles along M per group
    float alpha;
    int64_t tiles;       // size of the tile-id space (a multiple of XCDS * XCD_BLOCK)
    uint8_t* qcodes;     // QOUT: row-wise MXFP4 of the bf16 output, codes [M rows of qld bytes]
    uint8_t* qscales;    //       and scales [M x N/32]
    int64_t qld;         //       the code rows' pitch in bytes (>= N/2)
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
// scales (256 rows x 8 dwords each; scales moved in pairs take 4 dwords a
// row, staged scales 2)
constexpr int OFF_A = 0, OFF_B = 32768, OFF_AS = 65536, OFF_BS = 73728;
constexpr int STAGE_BYTES = 81920;
// DMA ops per thread per stage: 8 code moves (4 rows of each operand), 4
// A-scale moves (one byte each) or 2 (SA2: two bytes each), and 4 or 2
// (SA2) B-scale moves for 1D B scales, or 1 for 2D B scales (8 row groups
// of 32 per tile).  Staged scales (STG) take one dword move per operand
// whose scales are staged: 10 in all (the other operand's being 2D).
template <bool B2D, bool SA2>
constexpr int dma_per_stage() { return 8 + (SA2 ? 2 : 4) + (B2D ? 1 : (SA2 ? 2 : 4)); }

// 16-byte chunk swizzle of a 128-byte row: the rows an MFMA operand read
// touches at one chunk index land in distinct 16-byte bank groups whether
// the LDS serves 8 lanes (32 banks: rows r..r+7) or 16 lanes (64 banks: the
// even and the odd rows of r..r+15) of a ds_read_b128 per cycle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// LDS-DMA: every lane moves 16 bytes (or 1 byte, zero-extended to a dword)
// from base + voff to LDS byte address lds + 16 lane (or + 4 lane).  M0
// carries the wave's LDS base.  Register operands only; completion is
// awaited with an explicit s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma2(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma1(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}

// a value every lane holds alike, moved to scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;   // v_cvt_pk_bf16_f32: round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// SA2: the scales of a stage move two bytes per lane (global_load_lds_ushort),
// half the DMA instructions of one byte per lane.  It needs every pair of
// scale bytes 2-byte aligned: an even K / 32 and even scale pointers; with
// groups along K each tile's K window starts at an even chunk (Tile::head).
// QOUT: the epilogue also quantizes the bf16 output row-wise (1x32 blocks
// along N, round to nearest even), as the 1D quantizer would.
template <bool OUT_BF16, bool B2D, bool GK, bool GATHER, bool SA2, bool QOUT, bool STG>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmArgs p) {
    static_assert(!(GK && (B2D || GATHER)), "groups along K take 1D scales and no row index");
    static_assert(!STG || (!GATHER && (GK || B2D)), "staged scales: A without a row index; B 2D or staged");
    static_assert(!QOUT || (OUT_BF16 && !GK), "the quantized output is the bf16 output of groups along M");
    // 2 x 4 waves of 128 x 64
    constexpr int WM = 128, WN = 64, FM = 4, FN = WN / 32;
    constexpr int NJ = 2048 / NT;               // code (and scale) moves per operand per thread
    __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t KBA = p.lda, KBB = p.ldb;   // code row pitch of A and B (>= K / 2 bytes)
    const int64_t KS = p.K / 32;     // scale bytes per operand row

    // ---------------- group table ----------------
    // With fewer than 64 groups every wave keeps the offsets in its lanes
    // (lane g: off[g]) and, when groups split M, the first tile id of each
    // group (a prefix sum of ceil(n_g / BM) * tiles_n), so finding a tile's
    // group is a ballot and two lane reads, with no memory round trip.
    // The offsets come from the device and are trusted only this far: each
    // is clamped to [0, M] (groups along M) or [0, K] (along K), and a group
    // whose end lies below its start is empty, so malformed offsets can
    // neither store outside C nor read past the operands.
    const int32_t lim = GK ? (int32_t)p.K : (int32_t)p.M;
    auto clamp_off = [lim](int32_t v) { return min(max(v, 0), lim); };
    const bool table = p.G < 64;
    int32_t off_l = 0, first_l = 0;
    if (table) {
        if (lane <= p.G) off_l = clamp_off(p.off[lane]);
        if (!GK) {
            const int32_t next = __shfl_down(off_l, 1);
            const int32_t t = lane < p.G && next > off_l ? (next - off_l + BM - 1) / BM * p.tiles_n : 0;
            int32_t incl = t;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int32_t v = __shfl_up(incl, d);
                if (lane >= d) incl += v;
            }
            first_l = incl - t;                  // lane G: the total tile count
        } else if (STG) {
            // staged scales: group g's stages follow those of the groups
            // before it; first_l = the first stage of group `lane`
            const int32_t next = max(off_l, __shfl_down(off_l, 1));
            const int32_t t = lane < p.G && next > off_l ? (next / 32 - off_l / 32 + 7) / 8 : 0;
            int32_t incl = t;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int32_t v = __shfl_up(incl, d);
                if (lane >= d) incl += v;
            }
            first_l = incl - t;
        }
    }

    struct Tile {
        int32_t m0, m1, n0;      // output rows [m0, m1) and first output column
        int32_t g;               // group
        int32_t kc0, kc_last;    // first K chunk (of 32); last valid chunk relative to it
        int32_t nkt;             // K stages
        int32_t head;            // 1: chunk kc0 lies before the group (groups along K, SA2)
        int32_t sg;              // staged scales: the stage index of the tile's K stage 0
    };
    // (the host bounds M, N, K and the tile count to int32)
    const int32_t M32 = (int32_t)p.M, N32 = (int32_t)p.N, K32 = (int32_t)p.K;

    // tile id -> tile; false if the id is past the last tile
    auto decode = [&](int32_t L, Tile& t) -> bool {
        // XCD-aware remap of the position: 32 consecutive ids per XCD turn
        const int32_t xcd = L % XCDS, j = L / XCDS;
        int32_t id = (j / XCD_BLOCK) * (XCDS * XCD_BLOCK) + xcd * XCD_BLOCK + (j % XCD_BLOCK);
        int32_t g = -1, mb = 0, me = M32, kb = 0, ke = K32, mtiles, sg = 0;
        if (!GK) {
            if (table) {
                if (id >= __builtin_amdgcn_readlane(first_l, p.G)) return false;
                // the last group whose first tile is at or before id holds it
                const uint64_t below = __ballot(lane < p.G && first_l <= id);
                g = 63 - __builtin_clzll(below);
                id -= __builtin_amdgcn_readlane(first_l, g);
                mb = __builtin_amdgcn_readlane(off_l, g);
                me = max(mb, __builtin_amdgcn_readlane(off_l, g + 1));
            } else {
                // many groups: scan the offsets 64 at a time
                int32_t running = 0;
                for (int base = 0; base < p.G; base += 64) {
                    const int gg = base + lane;
                    int32_t t = 0, gb = 0, ge = 0;
                    if (gg < p.G) {
                        gb = clamp_off(p.off[gg]);
                        ge = max(gb, clamp_off(p.off[gg + 1]));
                        t = (ge - gb + BM - 1) / BM * p.tiles_n;
                    }
                    int32_t incl = t;
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const int32_t v = __shfl_up(incl, d);
                        if (lane >= d) incl += v;
                    }
                    const int32_t start = running + incl - t;
                    const uint64_t hit = __ballot(gg < p.G && id >= start && id < start + t);
                    if (hit) {
                        const int h = __builtin_ctzll(hit);
                        g = base + h;
                        id -= __builtin_amdgcn_readlane(start, h);
                        mb = __builtin_amdgcn_readlane(gb, h);
                        me = __builtin_amdgcn_readlane(ge, h);
                        break;
                    }
                    running += __builtin_amdgcn_readlane(incl, 63);
                }
                if (g < 0) return false;
            }
            mtiles = (me - mb + BM - 1) / BM;
        } else {
            const int32_t per = p.tiles_m * p.tiles_n;
            if (id / per >= p.G) return false;
            g = id / per;
            id -= g * per;
            mtiles = p.tiles_m;
            kb = table ? __builtin_amdgcn_readlane(off_l, g) : clamp_off(p.off[g]);
            ke = max(kb, table ? __builtin_amdgcn_readlane(off_l, g + 1) : clamp_off(p.off[g + 1]));
            if (STG) sg = __builtin_amdgcn_readlane(first_l, g);   // (staged: the host requires the table)
        }
        // grouped order inside the group: GROUP_M M-tiles x all N-tiles, m fastest
        const int32_t span = GROUP_M * p.tiles_n;
        const int32_t sgrp = id / span;
        const int32_t rem = id - sgrp * span;
        const int32_t gm = min(GROUP_M, mtiles - sgrp * GROUP_M);
        const int32_t nt = rem / gm;
        const int32_t mt = sgrp * GROUP_M + (rem - nt * gm);
        t.m0 = mb + mt * BM;
        t.m1 = min(me, t.m0 + BM);
        t.n0 = nt * BN;
        t.g = g;
        // groups along K with pair moves: the K window starts at the even
        // chunk at or below the group's first, so every scale pair is 2-byte
        // aligned; a chunk before the group (head) is masked like the tail
        t.head = GK && SA2 && !STG ? (kb / 32) & 1 : 0;
        t.sg = sg;
        t.kc0 = kb / 32 - t.head;
        t.kc_last = ke / 32 - t.kc0 - 1;
        t.nkt = ke > kb ? (ke / 32 - t.kc0 + BK / 32 - 1) / (BK / 32) : 0;
        return true;
    };

    // Persistent tile loop: in round r this workgroup takes position
    // r * P + w (w = its id) on even rounds and r * P + P - 1 - w on odd ones.
    // Tile ids within a group have equal cost, so the snake keeps the total
    // per workgroup even when groups differ in cost (weight gradient: K per
    // group follows the routing counts).
    const int32_t P = gridDim.x;
    const int32_t w = blockIdx.x;
    const int32_t tiles = (int32_t)p.tiles;
    auto find_tile = [&](int32_t& r, Tile& t) -> bool {
        for (;; ++r) {
            const int32_t L = r * P + ((r & 1) ? P - 1 - w : w);
            if (L >= tiles) return false;
            if (decode(L, t)) return true;
        }
    };
    // The A rows of this thread's DMA moves: entry j < NJ is code move j,
    // row t/8 + (NT/8) j; with A's scales moved in pairs (SA2, not staged)
    // entry NJ + j is scale move j, row 16 (j NW + w) + l/4 (w: wave, l: lane).
    constexpr int NR = SA2 && !STG ? NJ + 2 : NJ;
    auto load_rows = [&](const Tile& t, int32_t (&arow)[NR]) {
#pragma unroll
        for (int jj = 0; jj < NR; ++jj) {
            int32_t m = t.m0 + (jj < NJ ? (tid >> 3) + (NT / 8) * jj : 16 * ((jj - NJ) * NW + wave) + ((tid & 63) >> 2));
            if (m >= t.m1) m = t.m1 - 1;          // rows past the tile end are never stored
            arow[jj] = GATHER ? p.a_row_index[m] : m;
        }
    };

    // ---------------- per-thread DMA assignments ----------------
    // Code DMA j of thread t fills 16-byte slot t + NT j of an operand tile:
    // row t/8 + (NT/8) j, slot position pc = t % 8 of the row's 128 bytes, so
    // 8 lanes move one full 128-byte line.  Scale DMA j fills dword slot
    // t + NT j: the same row, scale position pc.  Byte offsets are 32-bit
    // (the host bounds every operand to 4 GiB).
    const int pc = tid & 7;
    const int a_chunk = pc ^ swz(tid >> 3);    // swz(t/8 + (NT/8) j) is the same for every j
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    // stage kt of tile t -> LDS buffer `buf`; chunks past the end are clamped
    // in range.  A stage's DMAs are numbered: A code rows (NJ), B code rows
    // (NJ), A scales (NJ / 2 pair moves or NJ byte moves), B scales (one 2D
    // group move, NJ / 2 pair moves or NJ byte moves).  issue_slot(m) issues those with number
    // p % 8 == m, so the main loop can spread a stage's DMAs over the eight
    // MFMA blocks of a K-quarter instead of issuing them in one burst.
    constexpr int NA_S = STG ? 1 : (SA2 ? NJ / 2 : NJ), NB_S = B2D || (STG && GK) ? 1 : (SA2 ? NJ / 2 : NJ);
    constexpr int NPARTS = 2 * NJ + NA_S + NB_S;
    static_assert(STG || NPARTS == dma_per_stage<B2D, SA2>(), "DMA count");
    static_assert(!STG || NPARTS == 2 * NJ + 2, "DMA count");
    // staged scales: wave w moves tile rows 32 w .. 32 w + 31 of a stage's
    // scales, two lanes a row (4 bytes each: one K half of the stage), from
    // stage t.sg + kt of the staged layout ([stage][row][8 bytes]); tile row r
    // lands at 8 r.  Stages past the tile's last repeat the last.
    auto staged_off = [&](const Tile& t, int kt, int32_t row, int64_t rows) {
        const uint32_t st = (uint32_t)(t.sg + min(kt, t.kc_last >> 3));
        return (st * (uint32_t)rows + (uint32_t)row) * 8u + (uint32_t)(tid & 1) * 4u;
    };
    auto issue_slot = [&](const Tile& t, const int32_t (&arow)[NR], int kt, int buf, int slot) {
        const uint32_t sb = lds_base + (uint32_t)buf * STAGE_BYTES;
        const uint8_t* bcodes = p.b_codes;
        const uint8_t* bscales = p.b_scales;
        if (!GK) {
            bcodes += (int64_t)t.g * p.N * KBB;
            bscales += (int64_t)t.g * (B2D ? (p.N / 32) * KS : p.N * KS);
        }
        auto nrow = [&](int jj) {
            const int32_t n = t.n0 + (tid >> 3) + (NT / 8) * jj;
            return (uint32_t)(n < N32 ? n : N32 - 1);       // rows past N are never stored
        };
#pragma unroll
        for (int part = slot; part < NPARTS; part += 8) {
            if (part < NJ) {
                const int jj = part;
                const uint32_t kc = (uint32_t)(t.kc0 + min(kt * 8 + a_chunk, t.kc_last));
                dma16(p.a_codes, (uint32_t)arow[jj] * (uint32_t)KBA + kc * 16, sb + OFF_A + jj * NT * 16 + wave * 1024);
            } else if (part < 2 * NJ) {
                const int jj = part - NJ;
                const uint32_t kc = (uint32_t)(t.kc0 + min(kt * 8 + a_chunk, t.kc_last));
                dma16(bcodes, nrow(jj) * (uint32_t)KBB + kc * 16, sb + OFF_B + jj * NT * 16 + wave * 1024);
            } else if (part < 2 * NJ + NA_S) {
                const int j = part - 2 * NJ;
                if (STG) {
                    int32_t m = t.m0 + 32 * wave + ((tid & 63) >> 1);
                    if (m >= t.m1) m = t.m1 - 1;
                    dma4(p.a_scales, staged_off(t, kt, m, p.M), sb + OFF_AS + wave * 256);
                } else if (SA2) {
                    // move j of wave w fills tile rows 16 (j NW + w) .. + 15,
                    // four lanes a row: lane l takes pair l % 4 of its row,
                    // so tile row r lands at 16 r (pair p at + 4 p) and an
                    // MFMA block's scale read is one contiguous 512-byte span;
                    // pairs past the end repeat the pair that holds the last
                    // chunk
                    const uint32_t kp = (uint32_t)(t.kc0 + min(kt * 8 + 2 * (pc & 3), t.kc_last & ~1));
                    dma2(p.a_scales, (uint32_t)arow[NJ + j] * (uint32_t)KS + kp, sb + OFF_AS + (j * NW + wave) * 256);
                } else {
                    const uint32_t ks = (uint32_t)(t.kc0 + min(kt * 8 + pc, t.kc_last));
                    dma1(p.a_scales, (uint32_t)arow[j] * (uint32_t)KS + ks, sb + OFF_AS + j * NT * 4 + wave * 256);
                }
            } else {
                const int j = part - 2 * NJ - NA_S;
                if (STG && GK) {
                    const int32_t n = t.n0 + 32 * wave + ((tid & 63) >> 1);
                    dma4(bscales, staged_off(t, kt, n < N32 ? n : N32 - 1, p.N), sb + OFF_BS + wave * 256);
                } else if (B2D) {
                    // wave w fetches row group w of the tile (8 groups of 32
                    // rows): lane l takes scale position l % 8 (SA2: pair
                    // l % 4), so the copies of the same 8 bytes coalesce into
                    // one line request (one group per wave instead of all 8 in
                    // every wave: 8x fewer requests)
                    int32_t grp = t.n0 / 32 + wave;
                    if (grp > N32 / 32 - 1) grp = N32 / 32 - 1;    // groups past N are never stored
                    if (SA2) {
                        const uint32_t kp = (uint32_t)(t.kc0 + min(kt * 8 + 2 * (pc & 3), t.kc_last & ~1));
                        dma2(bscales, (uint32_t)grp * (uint32_t)KS + kp, sb + OFF_BS + wave * 256);
                    } else {
                        const uint32_t ks = (uint32_t)(t.kc0 + min(kt * 8 + pc, t.kc_last));
                        dma1(bscales, (uint32_t)grp * (uint32_t)KS + ks, sb + OFF_BS + wave * 256);
                    }
                } else if (SA2) {
                    // as the A scales: tile row 16 (j NW + w) + l / 4
                    const int32_t n = t.n0 + 16 * (j * NW + wave) + ((tid & 63) >> 2);
                    const uint32_t kp = (uint32_t)(t.kc0 + min(kt * 8 + 2 * (pc & 3), t.kc_last & ~1));
                    dma2(bscales, (uint32_t)(n < N32 ? n : N32 - 1) * (uint32_t)KS + kp,
                         sb + OFF_BS + (j * NW + wave) * 256);
                } else {
                    const uint32_t ks = (uint32_t)(t.kc0 + min(kt * 8 + pc, t.kc_last));
                    dma1(bscales, nrow(j) * (uint32_t)KS + ks, sb + OFF_BS + j * NT * 4 + wave * 256);
                }
            }
        }
    };
    auto issue = [&](const Tile& t, const int32_t (&arow)[NR], int kt, int buf) {
#pragma unroll
        for (int slot = 0; slot < 8; ++slot) issue_slot(t, arow, kt, buf, slot);
    };

    const int lr = lane & 31;      // operand row within a 32-row MFMA block
    // K-quarter q of a stage (64 elements, one MFMA) takes chunk 4 h + q
    // in lane half h: any split of K works if both operands and their
    // scales agree, and this one keeps a lane's four scale bytes adjacent
    const int lh = lane >> 5;
    // operand rows w*128 + i*32 + lr share swz(lr) for every i, so a fragment
    // read is one per-lane base plus an immediate i * 4096
    const int sw = swz(lr);
    const uint32_t fb_b = OFF_B + (uint32_t)(wn * WN + lr) * 128;
    const uint32_t fb_a = OFF_A + (uint32_t)(wm * WM + lr) * 128;

    v16f acc[FN][FM];
    struct Frag { v8i b[FN]; v8i a[FM]; };
    // a row's four K-quarter scale bytes packed in one register (byte q:
    // K-quarter q); the MFMA's scale operand selects the byte
    struct Scl { uint32_t b[FN]; uint32_t a[FM]; };
    auto read_frag = [&](Frag& f, int buf, int q) {
        const uint8_t* sb = lds + buf * STAGE_BYTES + (((4 * lh + q) ^ sw) * 16);
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
    // the next stage's scales are read during the current stage's last
    // K-quarter and packed only after its MFMAs, when the reads have landed
    // Scale dword p of a row holds chunk p (one byte moves) or chunks 2 p
    // and 2 p + 1 (pair moves, SA2): lane half h takes dwords 4 h .. 4 h + 3
    // or 2 h, 2 h + 1.  B scales (1D or 2D) move in pairs along with A's.
    // A row's dwords are adjacent and the rows of an MFMA block are
    // consecutive, so each read below covers one contiguous span (no bank
    // conflicts), except 2D B scales, which every lane reads alike.
    constexpr bool SB2 = SA2;
    using ARaw = typename std::conditional<STG, uint32_t, typename std::conditional<SA2, uint2, uint4>::type>::type;
    using BRaw = typename std::conditional<STG && GK, uint32_t,
                                           typename std::conditional<SB2, uint2, uint4>::type>::type;
    struct SclRaw { BRaw b[FN]; ARaw a[FM]; };
    auto read_scl = [&](SclRaw& s, int buf) {
        const uint8_t* sb = lds + buf * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < FN; ++i)
            s.b[i] = B2D ? *(const BRaw*)(sb + OFF_BS + (wn * FN + i) * 256 + lh * (int)sizeof(BRaw))
                   : STG ? *(const BRaw*)(sb + OFF_BS + (wn * WN + i * 32 + lr) * 8 + lh * 4)
                   : SB2 ? *(const BRaw*)(sb + OFF_BS + (wn * WN + i * 32 + lr) * 16 + lh * 8)
                         : *(const BRaw*)(sb + OFF_BS + (wn * WN + i * 32 + lr) * 32 + lh * 16);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            s.a[i] = STG ? *(const ARaw*)(sb + OFF_AS + (wm * WM + i * 32 + lr) * 8 + lh * 4)
                   : SA2 ? *(const ARaw*)(sb + OFF_AS + (wm * WM + i * 32 + lr) * 16 + lh * 8)
                         : *(const ARaw*)(sb + OFF_AS + (wm * WM + i * 32 + lr) * 32 + lh * 16);
    };
    // byte q of the packed register: K-quarter q (a pair move leaves the
    // upper half of its dword zero)
    auto pack4 = [](const uint4& v) { return v.x | (v.y << 8) | (v.z << 16) | (v.w << 24); };
    auto pack2 = [](const uint2& v) { return v.x | (v.y << 16); };
    // groups along K with pair moves: a tile whose window starts one chunk
    // before its group clears that chunk's scale byte (K-quarter 0, lane half
    // 0) on both operands, so its products vanish as in the K tail
    auto head_mask = [&](Scl& s, int32_t head) {
        const uint32_t m = (head != 0 && lh == 0) ? 0xFFFFFF00u : 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < FN; ++i) s.b[i] &= m;
#pragma unroll
        for (int i = 0; i < FM; ++i) s.a[i] &= m;
    };
    auto pack = [&](Scl& s, const SclRaw& r) {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            if constexpr (STG && GK) s.b[i] = r.b[i];          // staged: the dword is the packed form
            else if constexpr (SB2) s.b[i] = pack2(r.b[i]);
            else s.b[i] = pack4(r.b[i]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if constexpr (STG) s.a[i] = r.a[i];
            else if constexpr (SA2) s.a[i] = pack2(r.a[i]);
            else s.a[i] = pack4(r.a[i]);
        }
    };

    // "every DMA but the newest stage's has landed"
    auto wait_all_but_one_stage = [] {
        if (STG) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        else if (B2D && SA2) asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
        else if (B2D) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
        else if (SA2) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    };
    static_assert(dma_per_stage<true, true>() == 11 && dma_per_stage<true, false>() == 13 &&
                  dma_per_stage<false, true>() == 12 && dma_per_stage<false, false>() == 16, "wait counts");
    // one MFMA block, optionally followed by one piece of the next read
    auto mma1 = [&](const Frag& f, const Scl& s, int q, bool tail, int m) {
        const int i = m / FM, jj = m % FM;
        const int sb = tail ? 0 : (int)s.b[i];
        const int sa = tail ? 0 : (int)s.a[jj];
        v16f& d = acc[i][jj];
        // the byte select is an immediate: q is a constant once inlined
        switch (q) {
        case 0: d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[i], f.a[jj], d, 4, 4, 0, sb, 0, sa); break;
        case 1: d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[i], f.a[jj], d, 4, 4, 1, sb, 1, sa); break;
        case 2: d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[i], f.a[jj], d, 4, 4, 2, sb, 2, sa); break;
        default: d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[i], f.a[jj], d, 4, 4, 3, sb, 3, sa); break;
        }
    };
    auto read_piece = [&](Frag& f, int buf, int q, int k) {
        const uint8_t* sb = lds + buf * STAGE_BYTES + (((4 * lh + q) ^ sw) * 16);
        const uint4 v = k < FN ? *(const uint4*)(sb + fb_b + k * 4096) : *(const uint4*)(sb + fb_a + (k - FN) * 4096);
        v8i& d = k < FN ? f.b[k] : f.a[k - FN];
        d = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    };
    // One K-quarter: 8 MFMA blocks (m = i * FM + jj), each followed by the
    // read of the next quarter's fragment piece whose last use it was, into
    // the same registers (B piece i is last used by block i FM + FM - 1, A
    // piece jj by block FM + jj), so a single fragment set suffices and every
    // read still has at least three MFMAs to land.  skip (wave-uniform): the
    // quarter lies wholly past the end of K, its MFMAs would add only zeros.
    auto no_extra = [](int) {};
    auto mma_rd = [&](Frag& f, const Scl& s, int q, bool tail, bool skip, int nbuf, int nq, auto&& extra) {
#pragma unroll
        for (int m = 0; m < FN * FM; ++m) {
            if (!skip) mma1(f, s, q, tail, m);
            extra(m);
            if (m == FM - 1) read_piece(f, nbuf, nq, 0);                 // B 0
            if (m >= FM) read_piece(f, nbuf, nq, FN + (m - FM));         // A m - FM
            if (m == FN * FM - 1) read_piece(f, nbuf, nq, 1);            // B 1
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---------------- epilogue: straight from the accumulators ----------------
    // Lane (lr, lh) of a 32 x 32 block holds output row lr, columns
    // 8 q + 4 lh + (0..3).  Two register swaps across lane groups
    // (v_permlane32_swap, v_permlane16_swap) regroup a block so that one
    // 16-byte store per lane writes 16 rows x 64 contiguous bytes, instead of
    // 32 rows x 16 bytes, which quarters the write requests.  The LDS is left
    // alone, so the next tile's first stages land meanwhile.
    auto swap32 = [](uint32_t& x, uint32_t& y) {   // x[32..63] <-> y[0..31]
        const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
        x = r[0];
        y = r[1];
    };
    auto swap16 = [](uint32_t& x, uint32_t& y) {   // x[16..31], x[48..63] <-> y[0..15], y[32..47]
        const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
        x = r[0];
        y = r[1];
    };
    // Stores go through a buffer resource spanning the tile's rows of C, so
    // a row or column outside C is dropped by the hardware range check
    // instead of a branch: every wave issues exactly EPI_STORES stores, which
    // lets the next tile's first barrier wait for its own loads only.
    // (QOUT adds one 8-byte code store and one scale-byte store per block)
    constexpr int EPI_STORES = OUT_BF16 ? FN * FM * (QOUT ? 4 : 2) : FN * FM * 4;
    auto epilogue = [&](const Tile& t) {
        constexpr int EB = OUT_BF16 ? 2 : 4;
        // (base and size are uniform: kept in scalar registers, the resource
        // needs no per-lane loop)
        uint8_t* cb = (uint8_t*)p.c + uniform64(((GK ? (int64_t)t.g * p.M : 0) + t.m0) * p.N * EB);
        // (QOUT may leave C out: a resource of size 0 drops every store)
        const int32_t nrec = __builtin_amdgcn_readfirstlane(QOUT && !p.c ? 0 : (t.m1 - t.m0) * N32 * EB);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(cb, (short)0, nrec, 0x00020000);
        // QOUT: the tile's rows of the code and scale outputs
        __amdgpu_buffer_rsrc_t qc_rsrc = rsrc, qs_rsrc = rsrc;
        if (QOUT) {
            uint8_t* qc = p.qcodes + uniform64((int64_t)t.m0 * p.qld);
            uint8_t* qs = p.qscales + uniform64((int64_t)t.m0 * (p.N / 32));
            qc_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                qc, (short)0, __builtin_amdgcn_readfirstlane((t.m1 - t.m0) * (int32_t)p.qld), 0x00020000);
            qs_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                qs, (short)0, __builtin_amdgcn_readfirstlane((t.m1 - t.m0) * (N32 / 32)), 0x00020000);
        }
        const float alpha = p.alpha;
        const int32_t col0 = t.n0 + wn * WN;            // first output column of this wave
        // the lane's coordinates pass through an empty asm so that the store
        // offsets are formed here: hoisted out of the tile loop they would
        // hold 16 registers through the K loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int elr = ln & 31, elh = ln >> 5;
        const int rh = elr >> 4;                        // (lane bits 0..3: the row rr within 16)
        const int32_t nrows = t.m1 - t.m0;
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        auto put = [&](int32_t row, int32_t col, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
            // row relative to the tile; out-of-range offsets (2 GiB) are dropped
            const uint32_t off = row < nrows && col < N32 ? (uint32_t)(row * N32 + col) * EB : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){v0, v1, v2, v3}, rsrc, off, 0, 0);
        };
        static_assert(FN == 2, "the bf16 stores pair the wave's two 32-column blocks");
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) {
            uint32_t G[FN][2][4];                          // bf16: block i, rows 16 h + rr, as stored
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const v16f& c = acc[i][jj];
                if (OUT_BF16) {
                    // P[q][d]: columns 8 q + 4 lh + 2 d, +1
                    uint32_t P[4][2];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int d = 0; d < 2; ++d)
                            P[q][d] = pack_bf16x2(c[4 * q + 2 * d] * alpha, c[4 * q + 2 * d + 1] * alpha);
                    if (QOUT) {
                        // The block of 32 columns of row lr is split over lanes
                        // lr and lr + 32 (16 values each: columns 8 q + 4 lh + e).
                        float w[16];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            w[4 * q + 0] = bf16lo(P[q][0]);
                            w[4 * q + 1] = bf16hi(P[q][0]);
                            w[4 * q + 2] = bf16lo(P[q][1]);
                            w[4 * q + 3] = bf16hi(P[q][1]);
                        }
                        uint32_t m = 0;
#pragma unroll
                        for (int e = 0; e < 16; ++e) m = max(m, __float_as_uint(w[e]) & 0x7FFFFFFFu);
                        const auto pm = __builtin_amdgcn_permlane32_swap(m, m, false, false);
                        m = max(pm[0], pm[1]);                      // own and partner half
                        const uint32_t byte = scale_byte_from_amax_bits(m);
                        const float scl = scale_operand(byte);
                        // d0: columns 4 lh + (0..3), 8 + 4 lh + (0..3); d1: the same + 16
                        uint32_t d0 = cvt8_rne(w, scl), d1 = cvt8_rne(w + 8, scl);
                        if (byte == 0xFFu) d0 = d1 = 0;             // non-finite block: codes 0
                        // lane lh = 0 holds block bytes (0 1 4 5 | 8 9 12 13), lh = 1
                        // (2 3 6 7 | 10 11 14 15): after the swap lh = 0 has bytes
                        // 0-7 and lh = 1 bytes 8-15 in (own, partner) pieces
                        swap32(d0, d1);
                        const uint32_t o0 = __builtin_amdgcn_perm(d1, d0, 0x05040100u);
                        const uint32_t o1 = __builtin_amdgcn_perm(d1, d0, 0x07060302u);
                        const int32_t qrow = wm * WM + jj * 32 + elr;
                        const int32_t qcol = col0 + i * 32;
                        const bool ok = qrow < nrows && qcol < N32;
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        __builtin_amdgcn_raw_buffer_store_b64(
                            (u32x2){o0, o1}, qc_rsrc,
                            ok ? (uint32_t)(qrow * (int32_t)p.qld + qcol / 2 + 8 * elh) : 0x80000000u, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b8(
                            (uint8_t)byte, qs_rsrc,
                            ok && elh == 0 ? (uint32_t)(qrow * (N32 / 32) + qcol / 32) : 0x80000000u, 0, 0);
                    }
                    // -> lane (lr, lh): P[0..1] columns 8 lh + (0..7), P[2..3] 16 + 8 lh + (0..7)
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        swap32(P[0][d], P[1][d]);
                        swap32(P[2][d], P[3][d]);
                    }
                    // -> first group: row rr, columns 16 rh + 8 lh + (0..7); second: row 16 + rr
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        swap16(P[0][d], P[2][d]);
                        swap16(P[1][d], P[3][d]);
                    }
                    // G[i][h]: row 16 h + rr, columns 32 i + 16 rh + 8 lh + (0..7)
                    G[i][0][0] = P[0][0]; G[i][0][1] = P[0][1]; G[i][0][2] = P[1][0]; G[i][0][3] = P[1][1];
                    G[i][1][0] = P[2][0]; G[i][1][1] = P[2][1]; G[i][1][2] = P[3][0]; G[i][1][3] = P[3][1];
                } else {
                    // Y[q]: columns 8 q + 4 lh + (0..3)
                    uint32_t Y[4][4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) Y[q][e] = __float_as_uint(c[4 * q + e] * alpha);
                    // -> Y[2h]: row rr, columns 16 h + 8 rh + 4 lh + (0..3); Y[2h+1]: row 16 + rr
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        swap16(Y[0][e], Y[1][e]);
                        swap16(Y[2][e], Y[3][e]);
                    }
                    // -> whole 128-byte row lines: lanes with bit 3 set trade
                    // their rows 0..7 of the left half (Y[2h]) for rows 8..15
                    // of the right half held 8 lanes away (a row rotate by 8,
                    // DPP), so one store writes 8 rows x 32 columns:
                    // Z[k]: row 8 k + (lane % 8), columns 16 b3 + 8 rh + 4 lh
                    const bool b3 = (ln & 8) != 0;
                    uint32_t Z[4][4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const uint32_t l8 = (uint32_t)__builtin_amdgcn_mov_dpp((int)Y[h][e], 0x128, 0xF, 0xF, false);
                            const uint32_t r8 = (uint32_t)__builtin_amdgcn_mov_dpp((int)Y[2 + h][e], 0x128, 0xF, 0xF, false);
                            Z[2 * h][e] = b3 ? r8 : Y[h][e];
                            Z[2 * h + 1][e] = b3 ? Y[2 + h][e] : l8;
                        }
                    }
                    const int32_t rb = wm * WM + jj * 32 + (ln & 7);
                    const int32_t col = col0 + i * 32 + (b3 ? 16 : 0) + 8 * rh + 4 * elh;
#pragma unroll
                    for (int k = 0; k < 4; ++k) put(rb + 8 * k, col, Z[k][0], Z[k][1], Z[k][2], Z[k][3]);
                }
            }
            if (OUT_BF16) {
                // whole 128-byte row lines from the wave's two blocks (64
                // bf16 columns): lanes with bit 3 set trade rows 0..7 of block
                // 0 for rows 8..15 of block 1 held 8 lanes away (DPP row
                // rotate by 8), so one store writes 8 rows x 64 columns
                const bool b3 = (ln & 8) != 0;
                const int32_t rb = wm * WM + jj * 32 + (ln & 7);
                const int32_t col = col0 + (b3 ? 32 : 0) + 16 * rh + 8 * elh;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t A[4], B[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t l8 = (uint32_t)__builtin_amdgcn_mov_dpp((int)G[0][h][e], 0x128, 0xF, 0xF, false);
                        const uint32_t r8 = (uint32_t)__builtin_amdgcn_mov_dpp((int)G[1][h][e], 0x128, 0xF, 0xF, false);
                        A[e] = b3 ? r8 : G[0][h][e];
                        B[e] = b3 ? G[1][h][e] : l8;
                    }
                    put(rb + 16 * h, col, A[0], A[1], A[2], A[3]);
                    put(rb + 16 * h + 8, col, B[0], B[1], B[2], B[3]);
                }
            }
        }
    };

    // ---------------- tile loop ----------------
    // The LDS ring runs on across tiles: at the barriers of the last two
    // stages of a tile (K stage count >= 2) the first two stages of the next
    // tile are issued, exactly as a tile's own stage kt+2 is issued at stage
    // kt's barrier, and the last K-quarter's reads already fetch the next
    // tile's first fragments.  The epilogue then overlaps those loads, and the
    // next tile starts its MFMAs without a prologue.
    Tile cur, nxt;
    int32_t arow[NR], narow[NR];
    int32_t round = 0;
    if (!find_tile(round, cur)) return;
    load_rows(cur, arow);
    Frag f0;
    Scl sc;
    SclRaw nsc;
    int par = 0;            // LDS buffer of the current tile's stage 0
    bool primed = false;    // its first two stages are issued and f0 / sc hold its first K-quarter
    for (;;) {
        // (every wave decodes the same tiles: the flags are uniform)
        int32_t nround = round + 1;
        const bool has_next = __builtin_amdgcn_readfirstlane((int)find_tile(nround, nxt)) != 0;
        if (has_next) load_rows(nxt, narow);
        const bool chain = __builtin_amdgcn_readfirstlane((int)(has_next && cur.nkt >= 2 && nxt.nkt >= 1)) != 0;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int jj = 0; jj < FM; ++jj)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.0f;
        if (cur.nkt > 0) {
            if (!primed) {
                // the previous tile's clamped past-the-end stage may still be
                // landing in the ring
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                issue(cur, arow, 0, par);
                issue(cur, arow, 1, par ^ 1);
                wait_all_but_one_stage();
                __builtin_amdgcn_s_barrier();
                read_frag(f0, par, 0);
                read_scl(nsc, par);
                pack(sc, nsc);
                if (GK && SA2 && !STG) head_mask(sc, cur.head);
            }
            // Stage kt+1's DMA was issued at stage kt-1's barrier, into the
            // buffer stage kt-1 had finished reading; at stage kt's barrier it
            // is the only DMA outstanding, so vmcnt(0) means it has landed.
            // At a chained tile's first barrier the previous tile's
            // EPI_STORES stores are the newest memory operations (without a
            // row gather nothing is loaded after them) and may stay in flight.
            // Only a tile's last stage can hold chunks past the end of K, so
            // only its copy of the stage computes the tail flags (they cost a
            // select per MFMA operand per K-quarter).
            auto stage = [&](int kt, auto first_c, auto last_c) {
                constexpr bool FIRST = decltype(first_c)::value;
                constexpr bool LAST = decltype(last_c)::value;
                const int buf = (kt & 1) ^ par;
                const int kcl = kt * 8 + 4 * lh;          // this lane's chunk in K-quarter 0
                // K-quarter q holds chunks kt 8 + q (lane half 0) and + 4: it
                // is all tail once the first is past the last chunk
                auto past = [&](int q) {
                    return LAST && __builtin_amdgcn_readfirstlane(kt * 8 + q - cur.kc_last) > 0;
                };
                mma_rd(f0, sc, 0, LAST && kcl > cur.kc_last, false, buf, 1, no_extra);
                mma_rd(f0, sc, 1, LAST && kcl + 1 > cur.kc_last, past(1), buf, 2, no_extra);
                mma_rd(f0, sc, 2, LAST && kcl + 2 > cur.kc_last, past(2), buf, 3, no_extra);
                if (FIRST) {
                    if (EPI_STORES == 16) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(32) lgkmcnt(0)" ::: "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                }
                __builtin_amdgcn_s_barrier();
                // Stage kt+2 of this tile, or at the last two stages the next
                // tile's stage 0 / 1 (chained), or else a clamped repeat of the
                // last stage that nothing reads.  Selected, not branched: a
                // branch here splits the loop body and the registers spill.
                const bool to_next = chain && kt + 2 >= cur.nkt;
                Tile t2;
                t2.n0 = to_next ? nxt.n0 : cur.n0;
                t2.g = to_next ? nxt.g : cur.g;
                t2.kc0 = to_next ? nxt.kc0 : cur.kc0;
                t2.kc_last = to_next ? nxt.kc_last : cur.kc_last;
                if (STG) {
                    t2.m0 = to_next ? nxt.m0 : cur.m0;
                    t2.m1 = to_next ? nxt.m1 : cur.m1;
                    t2.sg = to_next ? nxt.sg : cur.sg;
                }
                // The row select is pinned here, after the barrier's wait:
                // gathered row indices are ordinary loads, and the
                // compiler's wait for them lands before their first use.
                const uint64_t sel = __builtin_amdgcn_readfirstlane((int)to_next) ? ~0ull : 0ull;
                int32_t r2[NR];
#pragma unroll
                for (int jj = 0; jj < NR; ++jj)
                    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3"
                                 : "=v"(r2[jj]) : "v"(arow[jj]), "v"(narow[jj]), "s"(sel));
                // the DMAs of stage kt + 2 go out between the last K-quarter's
                // MFMA blocks (one or two after each), so a wave blocked on a
                // full memory pipeline stalls one block, not the whole burst
                const int kt2 = to_next ? kt + 2 - cur.nkt : kt + 2;
                read_scl(nsc, buf ^ 1);
                mma_rd(f0, sc, 3, LAST && kcl + 3 > cur.kc_last, past(3), buf ^ 1, 0,
                       [&](int m) { issue_slot(t2, r2, kt2, buf, m); });
                pack(sc, nsc);
                // the last stage packed the next tile's first scales (chained)
                if (GK && SA2 && !STG && LAST) head_mask(sc, chain ? nxt.head : 0);
            };
            // At a chained tile's first barrier the previous tile's
            // EPI_STORES stores are the newest memory operations (without a
            // row gather nothing is loaded after them) and may stay in flight.
            // (a one-stage tile takes the general first wait, vmcnt(0): it
            // also waits for the stores, which is correct, only slower)
            const int last = cur.nkt - 1;
            int kt = 0;
            if (!GATHER && primed && last > 0) {
                stage(0, std::true_type{}, std::false_type{});
                kt = 1;
            }
            for (; kt < last; ++kt) stage(kt, std::false_type{}, std::false_type{});
            stage(last, std::false_type{}, std::true_type{});
        }
        static_assert(EPI_STORES == 16 || EPI_STORES == 32, "first-barrier wait counts");
        epilogue(cur);
        if (!has_next) break;
        // unchained: the reads after the last barrier only fetched values
        // that are never used, so the next tile's prologue may refill both
        // buffers once the clamped stage still in flight has landed
        primed = chain;
        par = chain ? par ^ (cur.nkt & 1) : 0;
        cur = nxt;
#pragma unroll
        for (int jj = 0; jj < NR; ++jj) arow[jj] = narow[jj];
        round = nround;
    }
    // the clamped stages issued by the last tile may still be landing in
    // LDS: let them finish before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Validation shared by both entry points; fills everything but the outputs.
mx_status gemm_setup(const uint8_t* a_codes, int64_t a_ld, const uint8_t* a_scales, const int32_t* a_row_index,
                            const uint8_t* b_codes, int64_t b_ld, const uint8_t* b_scales, int scale_flags,
                            const int32_t* group_offsets, int32_t num_groups, int group_dim_k, int64_t M,
                            int64_t N, int64_t K, float alpha, GemmArgs& p, unsigned& grid) {
    if (M < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_ERR_SHAPE;
    if (scale_flags & ~(MX_SCALES_B_2D | MX_SCALES_STAGED)) return MX_ERR_UNSUPPORTED;
    const int b_scale_2d = scale_flags & MX_SCALES_B_2D;
    const bool staged = (scale_flags & MX_SCALES_STAGED) != 0;
    // code row pitch: 0 = K / 2 (contiguous rows); else at least K / 2 and
    // a multiple of 16 (every row starts 16-byte aligned)
    if (a_ld == 0) a_ld = K / 2;
    if (b_ld == 0) b_ld = K / 2;
    if (a_ld < K / 2 || b_ld < K / 2 || a_ld % 16 || b_ld % 16) return MX_ERR_SHAPE;
    if (num_groups < 1) return MX_ERR_SHAPE;
    if (group_dim_k != 0 && group_dim_k != 1) return MX_ERR_SHAPE;
    if (group_dim_k == 1 && (b_scale_2d || a_row_index)) return MX_ERR_UNSUPPORTED;
    // staged scales: groups along K need the in-register group table (fewer
    // than 64 groups); groups along M take them for A with 2D B scales and
    // no row index
    if (staged && group_dim_k == 1 && num_groups >= 64) return MX_ERR_UNSUPPORTED;
    if (staged && group_dim_k == 0 && (!b_scale_2d || a_row_index)) return MX_ERR_UNSUPPORTED;
    if (!group_offsets) return MX_ERR_NULL;
    if (M == 0) return MX_OK;
    if (!a_codes || !a_scales || !b_codes || !b_scales) return MX_ERR_NULL;
    if (!aligned16(a_codes) || !aligned16(b_codes)) return MX_ERR_ALIGN;
    // staged scales move as dwords
    if (staged && (((uintptr_t)a_scales & 3) || (group_dim_k == 1 && ((uintptr_t)b_scales & 3))))
        return MX_ERR_ALIGN;
    // operand bytes are addressed by 32-bit offsets from the operand's (or
    // the B group's) base: each must span at most 4 GiB.  With a row index
    // the caller keeps the indexed rows within that range.
    const int64_t lim = 0xFFFFFFFFLL;
    if (N * b_ld > lim) return MX_ERR_SHAPE;
    if (!a_row_index && M * a_ld > lim) return MX_ERR_SHAPE;
    // tile coordinates are 32-bit
    if (M > 0x7FFFFF00LL || N > 0x7FFFFF00LL || K > 0x7FFFFF00LL) return MX_ERR_SHAPE;
    // staged scales are addressed by 32-bit offsets too: at most K/256 + G
    // stages of 8 bytes per row
    if (staged && (K / 256 + num_groups + 1) * 8 * (group_dim_k == 1 ? max(M, N) : M) > lim) return MX_ERR_SHAPE;

    p = GemmArgs{};
    p.a_codes = a_codes;
    p.a_scales = a_scales;
    p.a_row_index = a_row_index;
    p.b_codes = b_codes;
    p.b_scales = b_scales;
    p.off = group_offsets;
    p.M = M;
    p.N = N;
    p.K = K;
    p.lda = a_ld;
    p.ldb = b_ld;
    p.G = num_groups;
    p.b_scale_2d = b_scale_2d ? 1 : 0;
    p.staged = staged ? 1 : 0;
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
    if (tiles > 0x7FFF0000) return MX_ERR_SHAPE;
    p.tiles = tiles;
    // persistent: one workgroup per CU (the ring takes all of its LDS)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    grid = (unsigned)min(tiles, (int64_t)cus);
    return MX_OK;
}

// groups split M: pick the instantiation for the B scale kind, the row gather
// and the A-scale move width
template <bool BF, bool QOUT>
void launch_m(const GemmArgs& p, unsigned grid, hipStream_t s) {
    const dim3 gd(grid), bd(NT);
    const bool gather = p.a_row_index != nullptr;
    const bool sa2 = (p.K / 32) % 2 == 0 && ((uintptr_t)p.a_scales & 1) == 0 && ((uintptr_t)p.b_scales & 1) == 0;
#define MX_GEMM_LAUNCH(B2, GA, S2) hipLaunchKernelGGL((gemm_kernel<BF, B2, false, GA, S2, QOUT, false>), gd, bd, 0, s, p)
#define MX_GEMM_S(B2, GA) \
    do { if (sa2) MX_GEMM_LAUNCH(B2, GA, true); else MX_GEMM_LAUNCH(B2, GA, false); } while (0)
#define MX_GEMM_G(B2) \
    do { if (gather) MX_GEMM_S(B2, true); else MX_GEMM_S(B2, false); } while (0)
    if (p.staged) {
        // staged A scales (2D B, no row index)
        if (sa2) hipLaunchKernelGGL((gemm_kernel<BF, true, false, false, true, QOUT, true>), gd, bd, 0, s, p);
        else hipLaunchKernelGGL((gemm_kernel<BF, true, false, false, false, QOUT, true>), gd, bd, 0, s, p);
    } else if (p.b_scale_2d) {
        MX_GEMM_G(true);
    } else {
        MX_GEMM_G(false);
    }
#undef MX_GEMM_G
#undef MX_GEMM_S
#undef MX_GEMM_LAUNCH
}

}  // namespace

extern "C" mx_status mx_grouped_gemm(const uint8_t* a_codes, int64_t a_ld, const uint8_t* a_scales,
                                     const int32_t* a_row_index, const uint8_t* b_codes, int64_t b_ld,
                                     const uint8_t* b_scales, int b_scale_2d,
                                     const int32_t* group_offsets, int32_t num_groups, int group_dim_k, int64_t M,
                                     int64_t N, int64_t K, float alpha, void* c, mx_dtype ct, mx_stream stream) {
    if (ct != MX_F32 && ct != MX_BF16) return MX_ERR_DTYPE;
    GemmArgs p;
    unsigned grid = 0;
    const mx_status st = gemm_setup(a_codes, a_ld, a_scales, a_row_index, b_codes, b_ld, b_scales, b_scale_2d,
                                    group_offsets, num_groups, group_dim_k, M, N, K, alpha, p, grid);
    if (st != MX_OK || M == 0) return st;
    if (!c) return MX_ERR_NULL;
    if (!aligned16(c)) return MX_ERR_ALIGN;
    p.c = c;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (group_dim_k == 1) {
        const dim3 gd(grid), bd(NT);
        const bool sa2 = (p.K / 32) % 2 == 0 && ((uintptr_t)p.a_scales & 1) == 0 && ((uintptr_t)p.b_scales & 1) == 0;
        if (p.staged) {
            if (ct == MX_BF16) hipLaunchKernelGGL((gemm_kernel<true, false, true, false, false, false, true>), gd, bd, 0, s, p);
            else hipLaunchKernelGGL((gemm_kernel<false, false, true, false, false, false, true>), gd, bd, 0, s, p);
        } else if (ct == MX_BF16) {
            if (sa2) hipLaunchKernelGGL((gemm_kernel<true, false, true, false, true, false, false>), gd, bd, 0, s, p);
            else hipLaunchKernelGGL((gemm_kernel<true, false, true, false, false, false, false>), gd, bd, 0, s, p);
        } else {
            if (sa2) hipLaunchKernelGGL((gemm_kernel<false, false, true, false, true, false, false>), gd, bd, 0, s, p);
            else hipLaunchKernelGGL((gemm_kernel<false, false, true, false, false, false, false>), gd, bd, 0, s, p);
        }
    } else if (ct == MX_BF16) {
        launch_m<true, false>(p, grid, s);
    } else {
        launch_m<false, false>(p, grid, s);
    }
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

extern "C" mx_status mx_grouped_gemm_q(const uint8_t* a_codes, int64_t a_ld, const uint8_t* a_scales,
                                       const int32_t* a_row_index, const uint8_t* b_codes, int64_t b_ld,
                                       const uint8_t* b_scales, int b_scale_2d,
                                       const int32_t* group_offsets, int32_t num_groups, int64_t M, int64_t N,
                                       int64_t K, float alpha, void* c, uint8_t* c_codes, int64_t c_codes_ld,
                                       uint8_t* c_scales, mx_stream stream) {
    GemmArgs p;
    unsigned grid = 0;
    const mx_status st = gemm_setup(a_codes, a_ld, a_scales, a_row_index, b_codes, b_ld, b_scales, b_scale_2d,
                                    group_offsets, num_groups, 0, M, N, K, alpha, p, grid);
    if (st != MX_OK || M == 0) return st;
    if (!c_codes || !c_scales) return MX_ERR_NULL;
    if (c_codes_ld == 0) c_codes_ld = N / 2;
    if (c_codes_ld < N / 2) return MX_ERR_SHAPE;
    if ((c && !aligned16(c)) || !aligned16(c_codes) || c_codes_ld % 16) return MX_ERR_ALIGN;
    // the code and scale outputs are addressed by 32-bit offsets per tile
    if (M * c_codes_ld > 0xFFFFFFFFLL) return MX_ERR_SHAPE;
    p.c = c;
    p.qcodes = c_codes;
    p.qld = c_codes_ld;
    p.qscales = c_scales;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    launch_m<true, true>(p, grid, s);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}
