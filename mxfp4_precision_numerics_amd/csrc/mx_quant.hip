// mx_quant.hip -- RHT, 1x32 / 32x32 MXFP4 quantization and dequantization
// kernels for gfx950, and their C-ABI entry points (include/mx.h).
//
// The kernels stream HBM (the RTNE ones are bound by it; with SR or the RHT
// the arithmetic binds first).  Lane mappings are chosen so that every
// global load and store of a wave is a contiguous run:
//   row-wise 1D / RHT: a quad of lanes owns one 32-block (8 elements per
//     lane, one 16-byte bf16 load), a wave covers 16 consecutive blocks; the
//     RHT's stages 8 and 16 cross lanes through DPP quad permutes; the lane's
//     8 elements take exactly one Philox call when rounding stochastically.
//   column-wise 1D: a persistent workgroup streams a contiguous run of
//     tiles of 256 padded tokens x 64 columns through LDS (128-byte row
//     reads, the next tile prefetched into registers while the current one
//     is quantized; the source rows of a block row are resolved once); a
//     thread takes 32 tokens of one column from LDS so the RHT and the block
//     amax stay in-lane, and codes are regrouped in LDS so each column's
//     tile leaves as one 128-byte run of the token-contiguous layout.
//   2D: a workgroup owns up to 8 x 8 tiles (256 x 256) and walks its tile
//     rows; lanes read 64 contiguous bytes of one tile row, the tile amax is
//     reduced across lanes and waves, and the transposed codes are regrouped
//     through LDS so each column leaves as one contiguous run.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/mx.h"
#include "mx_device.h"

using namespace mx;

// ===========================================================================
// Row-wise 1x32 quantization (optionally with the RHT).
// ===========================================================================
constexpr int ROW_UNROLL = 4;   // blocks per quad per loop trip (loads in flight)

// Code rows may be padded (PITCH > 0): block blk is block b of row r with
// blk = r * bpr + b, and its 16 code bytes go to codes + r * ld + 16 b
// = codes + 16 blk + r * pad, pad = ld - 16 bpr.
struct RowPitch {
    int64_t bpr;        // blocks per row (cols / 32)
    double inv_bpr;     // 1 / bpr
    int64_t pad;        // bytes between the end of a code row and the next row
    int64_t ld;         // bytes from one code row to the next
    int64_t step_rows;  // PITCH 2: the grid stride in blocks, as whole rows
    int64_t step_rem;   //          and the blocks left over
    uint32_t srows;     // 0: row-major scales; else the staged order with srows rows:
                        // block b of row r -> byte ((b / 8) srows + r) 8 + b % 8 (the host
                        // keeps the staged array below 4 GiB, so 32-bit offsets)
};

// row = floor(blk / bpr) from the double quotient, which is within one of it
// for any index below 2^53, and one correction step
__device__ __forceinline__ void split_block(int64_t blk, const RowPitch& rp, int64_t& row, int64_t& b) {
    row = (int64_t)((double)blk * rp.inv_bpr);
    b = blk - row * rp.bpr;
    if (b < 0) {
        --row;
        b += rp.bpr;
    } else if (b >= rp.bpr) {
        ++row;
        b -= rp.bpr;
    }
}

// PITCH: 0 unpadded rows; 1 padded rows of any width; 2 padded rows of at
// least 64 blocks, so a trip's 64 blocks cross at most one row end
template <bool BF16, bool RHT, bool SR, int PITCH>
__device__ __forceinline__ void q1d_row_body(const void* __restrict__ x, int64_t nblocks, uint32_t mask,
                                             uint32_t k0, uint32_t k1, uint32_t stream_id,
                                             uint64_t index_base, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales, RowPitch rp) {
    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    // per-lane sign words for the RHT: lane q holds block elements 8q..8q+7
    const uint32_t m8 = (mask >> (8 * q)) & 0xFFu;
    uint32_t sgn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sgn[e] = ((m8 >> e) & 1u) << 31;
    // PITCH 2: the wave's first block of the trip as (row0, b0), wave-uniform,
    // advanced by the grid stride with integer steps
    int64_t row0 = 0, b0 = 0;
    if (PITCH == 2) split_block(wave * 16 * ROW_UNROLL, rp, row0, b0);

    for (int64_t base = wave * 16 * ROW_UNROLL; base < nblocks; base += nwaves * 16 * ROW_UNROLL) {
        const int32_t bpr32 = (int32_t)rp.bpr;   // (the host bounds bpr to int32)
        // PITCH: the quad's first block split into (row, b) once per trip,
        // r = floor(blk / bpr) from the double quotient, which is within one
        // of it for any index below 2^53, and one correction step; the later
        // blocks step b by 16 and carry into the row
        int32_t pb = 0;
        int64_t pofs = 0;
        if (PITCH == 1) {
            int64_t row, b;
            const int64_t blk = base + (lane >> 2);
            split_block(blk, rp, row, b);
            pb = (int32_t)b;
            pofs = blk * 16 + row * rp.pad;
        }
        // PITCH 2: block base + o lies in row row0 while o < bpr - b0, else in
        // the next row; its codes are o * 16 (+ pad) bytes past row0's block b0
        uint8_t* const cbase = codes + (PITCH == 2 ? row0 * rp.ld + b0 * 16 : 0);
        const int32_t thr = (int32_t)(rp.bpr - b0);
        // With SR or the RHT (arithmetic-heavy) the trip's loads are
        // unconditional, so all of them are in flight before the first is
        // used: a block past the end reads the last block instead (a quad's
        // values only feed its own block, whose codes and scale are not
        // stored).  Plain RTNE keeps one guarded load at a time, which
        // measured 3% faster for it (65536 x 2880 bf16).
        constexpr bool PIPE = SR || RHT;
        float v[ROW_UNROLL][8];
#pragma unroll
        for (int u = 0; u < ROW_UNROLL; ++u) {
            const int64_t blk = base + u * 16 + (lane >> 2);
            const int64_t blc = blk < nblocks ? blk : nblocks - 1;
            if (!PIPE && blk >= nblocks) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
            } else if (BF16) {
                const uint4 w = *((const uint4*)((const uint8_t*)x + blc * 64) + q);
                v[u][0] = bf16lo(w.x); v[u][1] = bf16hi(w.x);
                v[u][2] = bf16lo(w.y); v[u][3] = bf16hi(w.y);
                v[u][4] = bf16lo(w.z); v[u][5] = bf16hi(w.z);
                v[u][6] = bf16lo(w.w); v[u][7] = bf16hi(w.w);
            } else {
                const uint4* p = (const uint4*)((const uint8_t*)x + blc * 128) + 2 * q;
                const uint4 a = p[0], b = p[1];
                v[u][0] = __uint_as_float(a.x); v[u][1] = __uint_as_float(a.y);
                v[u][2] = __uint_as_float(a.z); v[u][3] = __uint_as_float(a.w);
                v[u][4] = __uint_as_float(b.x); v[u][5] = __uint_as_float(b.y);
                v[u][6] = __uint_as_float(b.z); v[u][7] = __uint_as_float(b.w);
            }
        }
        // every lane of a quad holds its block's scale byte; after the trip,
        // lane q stores the byte of step u = q (64 consecutive blocks per wave)
        static_assert(ROW_UNROLL == 4, "one scale store per quad lane");
        uint32_t sbyte[ROW_UNROLL];
        const uint64_t g0 = SR ? (index_base + (uint64_t)(base + (lane >> 2)) * 32 + (uint64_t)q * 8) >> 3 : 0;
#pragma unroll
        for (int u = 0; u < ROW_UNROLL; ++u) {
            const int64_t blk = base + u * 16 + (lane >> 2);
            if (PITCH == 1 && u > 0) {
                pb += 16;
                pofs += 256;
                while (pb >= bpr32) {
                    pb -= bpr32;
                    pofs += rp.pad;
                }
            }
            float* t = v[u];
            if (RHT) {
#pragma unroll
                for (int e = 0; e < 8; ++e) t[e] = __uint_as_float(__float_as_uint(t[e]) ^ sgn[e]);
                rht32_quad(t, q);
            }
            uint32_t am = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(t[e]) & 0x7FFFFFFFu);
            am = quad_max_u(am);
            const uint32_t byte = scale_byte_from_amax_bits(am);
            const float sc = scale_operand(byte);
            uint32_t packed;
            if (SR) {
                // counter of this lane's 8 elements: (index_base + 32 blk + 8 q) / 8,
                // stepping by 64 per u (a multiple of 8 added before the shift)
                const uint64_t g = g0 + 64u * (uint32_t)u;
                const u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u, k0, k1);
                packed = cvt8_sr(t, sc, r);
            } else {
                packed = cvt8_rne(t, sc);
            }
            if (byte == 0xFFu) packed = 0;   // non-finite block: codes are 0
            sbyte[u] = byte;
            if (blk < nblocks) {
                if (PITCH == 2) {
                    const int32_t o = u * 16 + (lane >> 2);
                    const uint32_t rel = (uint32_t)o * 16u + (o >= thr ? (uint32_t)rp.pad : 0u);
                    *((uint32_t*)(cbase + rel) + q) = packed;
                } else {
                    const int64_t cofs = PITCH ? pofs : blk * 16;
                    *((uint32_t*)(codes + cofs) + q) = packed;
                }
            }
        }
        {
            const int64_t blk = base + q * 16 + (lane >> 2);
            const uint32_t byte = q == 0 ? sbyte[0] : q == 1 ? sbyte[1] : q == 2 ? sbyte[2] : sbyte[3];
            if (blk < nblocks) {
                if (rp.srows) {
                    // staged scales: the block's row and its block in the row
                    int64_t srow, sb;
                    if (PITCH == 2) {
                        const int32_t o = q * 16 + (lane >> 2);
                        srow = row0 + (o >= thr ? 1 : 0);
                        sb = o >= thr ? o - thr : b0 + o;
                    } else {
                        split_block(blk, rp, srow, sb);
                    }
                    scales[((uint32_t)(sb >> 3) * rp.srows + (uint32_t)srow) * 8u + (uint32_t)(sb & 7)] = (uint8_t)byte;
                } else {
                    scales[blk] = (uint8_t)byte;
                }
            }
        }
        if (PITCH == 2) {
            b0 += rp.step_rem;
            row0 += rp.step_rows;
            if (b0 >= rp.bpr) {
                b0 -= rp.bpr;
                ++row0;
            }
        }
    }
}

template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(256) void q1d_row_kernel(const void* __restrict__ x, int64_t nblocks,
                                                      uint32_t mask, uint32_t k0, uint32_t k1,
                                                      uint32_t stream_id, uint64_t index_base,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, RowPitch rp) {
    q1d_row_body<BF16, RHT, SR, 0>(x, nblocks, mask, k0, k1, stream_id, index_base, codes, scales, rp);
}

// the same with padded code rows
template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(256) void q1d_row_kernel_p(const void* __restrict__ x, int64_t nblocks,
                                                        uint32_t mask, uint32_t k0, uint32_t k1,
                                                        uint32_t stream_id, uint64_t index_base,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, RowPitch rp) {
    q1d_row_body<BF16, RHT, SR, 1>(x, nblocks, mask, k0, k1, stream_id, index_base, codes, scales, rp);
}

// the same with padded code rows of at least 64 blocks
template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(256) void q1d_row_kernel_w(const void* __restrict__ x, int64_t nblocks,
                                                        uint32_t mask, uint32_t k0, uint32_t k1,
                                                        uint32_t stream_id, uint64_t index_base,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, RowPitch rp) {
    q1d_row_body<BF16, RHT, SR, 2>(x, nblocks, mask, k0, k1, stream_id, index_base, codes, scales, rp);
}

// ===========================================================================
// Stand-alone RHT (fp32 output), same quad mapping.
// ===========================================================================
template <bool BF16, bool INV>
__global__ __launch_bounds__(256) void rht_kernel(const void* __restrict__ x, int64_t nblocks, uint32_t mask,
                                                  float* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const uint32_t m8 = (mask >> (8 * q)) & 0xFFu;
    for (int64_t base = wave * 16; base < nblocks; base += nwaves * 16) {
        const int64_t blk = base + (lane >> 2);
        float t[8];
        if (blk < nblocks) {
            if (BF16) {
                const uint4 w = *((const uint4*)((const uint8_t*)x + blk * 64) + q);
                t[0] = bf16lo(w.x); t[1] = bf16hi(w.x); t[2] = bf16lo(w.y); t[3] = bf16hi(w.y);
                t[4] = bf16lo(w.z); t[5] = bf16hi(w.z); t[6] = bf16lo(w.w); t[7] = bf16hi(w.w);
            } else {
                const uint4* p = (const uint4*)((const uint8_t*)x + blk * 128) + 2 * q;
                const uint4 a = p[0], b = p[1];
                t[0] = __uint_as_float(a.x); t[1] = __uint_as_float(a.y);
                t[2] = __uint_as_float(a.z); t[3] = __uint_as_float(a.w);
                t[4] = __uint_as_float(b.x); t[5] = __uint_as_float(b.y);
                t[6] = __uint_as_float(b.z); t[7] = __uint_as_float(b.w);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = 0.0f;
        }
        if (!INV) {
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = __uint_as_float(__float_as_uint(t[e]) ^ (((m8 >> e) & 1u) << 31));
        }
        rht32_quad(t, q);
        if (INV) {
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = __uint_as_float(__float_as_uint(t[e]) ^ (((m8 >> e) & 1u) << 31));
        }
        if (blk < nblocks) {
            uint4* o = (uint4*)(y + blk * 32) + 2 * q;
            o[0] = make_uint4(__float_as_uint(t[0]), __float_as_uint(t[1]), __float_as_uint(t[2]), __float_as_uint(t[3]));
            o[1] = make_uint4(__float_as_uint(t[4]), __float_as_uint(t[5]), __float_as_uint(t[6]), __float_as_uint(t[7]));
        }
    }
}

// ===========================================================================
// Column-wise, grouped 1x32 quantization (blocks run down the token axis of
// one group; output transposed so tokens are contiguous).
//
// A workgroup quantizes tiles of 8 consecutive padded 32-token blocks x 64
// columns.  The tile's token rows are read with coalesced 16-byte loads into
// LDS; each thread then takes two adjacent columns of one block from LDS
// (32 tokens each, so the RHT and the amax stay in-lane); the codes are
// regrouped in LDS so that every column's 8 blocks leave as one contiguous
// 128-byte run of the token-contiguous output.
// ===========================================================================
constexpr int COL_MAX_GROUPS = 4096;
constexpr int CT_BLOCKS = 8;                 // padded 32-token blocks per tile
constexpr int CT_COLS = 64;                  // columns per tile
constexpr int CT_OUT_PITCH = CT_BLOCKS * 16 + 16;   // LDS bytes per column of staged codes

template <bool BF16>
struct ColTile {
    static constexpr int EB = BF16 ? 2 : 4;
    static constexpr int ROWB = CT_COLS * EB;                 // bytes of one token row of the tile
    static constexpr int BSTRIDE = 32 * ROWB + 128;           // LDS bytes per block (+128: next block
                                                              // starts in the other half of the banks)
    static constexpr int TILE = CT_BLOCKS * BSTRIDE;
};

// ROWQ (the dual form): the same tile is also quantized row-wise (1x32
// blocks along the columns, no RHT; 1 = RTNE, 2 = SR with its own stream
// and index base), as mx_quantize_1d(block_axis = 1) would quantize the
// grouped rows: one read of x feeds both layouts.
struct ColArgs {
    const void* x;
    int64_t cols;
    const int32_t* off;
    int num_groups;
    const int32_t* ridx;
    int64_t npos;
    int64_t kp, col_tiles;
    int vec;
    uint32_t mask, k0, k1, stream_id;
    uint64_t index_base;
    uint8_t* codes;
    uint8_t* scales;
    // ROWQ: the row-wise outputs
    uint8_t* row_codes;
    int64_t row_ld;
    uint8_t* row_scales;
    uint32_t row_stream_id;
    uint64_t row_index_base;
    // scales in the staged layout (each group's blocks start a new stage of 8)
    int staged;
    // blocks per group padding unit: 1 (groups padded to 32 tokens) or 8 (256)
    int pad_blocks;
    // ROWQ: 0, row-major row-wise scales; else staged with this many rows
    // (block b of grouped row r at byte ((b / 8) row_srows + r) 8 + b % 8)
    uint32_t row_srows;
};

template <bool BF16, bool RHT, bool SR, int ROWQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BF16 ? 3 : 2))) void q1d_col_kernel(ColArgs a) {
    const void* __restrict__ x = a.x;
    const int64_t cols = a.cols;
    const int32_t* __restrict__ off = a.off;
    const int num_groups = a.num_groups;
    const int32_t* __restrict__ ridx = a.ridx;
    const int64_t npos = a.npos, kp = a.kp, col_tiles = a.col_tiles;
    const int vec = a.vec;
    const uint32_t mask = a.mask, k0 = a.k0, k1 = a.k1, stream_id = a.stream_id;
    const uint64_t index_base = a.index_base;
    uint8_t* __restrict__ codes = a.codes;
    uint8_t* __restrict__ scales = a.scales;
    using TL = ColTile<BF16>;
    constexpr int CH = TL::ROWB / 16;                       // 16-byte chunks per tile row
    constexpr int NLD = CT_BLOCKS * 32 * CH / 256;           // chunks per thread per tile
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* tile = smem;                                          // TL::TILE bytes
    int32_t* pstart = (int32_t*)(smem + TL::TILE);                 // num_groups + 1
    int32_t* sstart = pstart + num_groups + 1;                     // staged: num_groups + 1
    __shared__ int32_t wave_sum[4], wave_ssum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // padded start (in 32-token blocks) of every group: block-wide scan of
    // ceil32(n_g) / 32, each thread summing a contiguous chunk of groups;
    // staged scales also need each group's first stage (a scan of
    // ceil(blocks / 8))
    const bool staged = a.staged != 0;
    {
        const int chunk = (num_groups + 255) / 256;
        const int g0 = min(num_groups, tid * chunk), g1 = min(num_groups, g0 + chunk);
        int32_t local = 0, slocal = 0;
        const int32_t pu = a.pad_blocks;
        auto padded_blocks = [&](int g) {
            const int32_t nb = (off[g + 1] - off[g] + 31) >> 5;
            return pu == 8 ? (nb + 7) & ~7 : nb;
        };
        for (int g = g0; g < g1; ++g) {
            const int32_t nb = padded_blocks(g);
            local += nb;
            slocal += (nb + 7) >> 3;
        }
        int32_t incl = local, sincl = slocal;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t v = __shfl_up(incl, d), sv = __shfl_up(sincl, d);
            if (lane >= d) {
                incl += v;
                sincl += sv;
            }
        }
        if (lane == 63) {
            wave_sum[wave] = incl;
            wave_ssum[wave] = sincl;
        }
        __syncthreads();
        int32_t run = incl - local, srun = sincl - slocal;
        for (int w = 0; w < wave; ++w) {
            run += wave_sum[w];
            srun += wave_ssum[w];
        }
        for (int g = g0; g < g1; ++g) {
            const int32_t nb = padded_blocks(g);
            pstart[g] = run;
            run += nb;
            if (staged) sstart[g] = srun;
            srun += (nb + 7) >> 3;
        }
        if (tid == 255) {
            pstart[num_groups] = run;
            if (staged) sstart[num_groups] = srun;
        }
        __syncthreads();
    }
    // The offsets come from the device and are trusted only this far: the
    // blocks written stop at the capacity kp, and a token position outside
    // [0, npos) is read as padding, so malformed offsets can neither write
    // past the outputs nor read past x (or the row index).
    const int64_t kp_blocks = kp >> 5;
    const int64_t nblk_total = min((int64_t)pstart[num_groups], kp_blocks);

    // Token range of the tile's 8 blocks: lane b < 8 of every wave resolves
    // block b (its group by binary search over pstart); n = -1 marks a block
    // past the padded total.
    auto block_info = [&](int64_t pb0, int64_t& t0, int32_t& n) {
        t0 = 0;
        n = -1;
        const int64_t pb = pb0 + lane;
        if (lane < CT_BLOCKS && pb < nblk_total) {
            int lo = 0, hi = num_groups - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pstart[mid] <= pb) lo = mid; else hi = mid - 1;
            }
            t0 = (int64_t)off[lo] + (pb - pstart[lo]) * 32;
            n = (int32_t)max((int64_t)0, min(min((int64_t)32, (int64_t)off[lo + 1] - t0), npos - t0));
            if (t0 < 0) n = 0;
        }
    };
    auto bcast64 = [](int64_t v, int src) {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, src);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), src);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    // chunk k of this thread: block, row in block, 16-byte chunk in the row
    auto chunk_b = [&](int k) { return BF16 ? k : (k >> 1); };
    auto chunk_j = [&](int k) { return BF16 ? (tid >> 3) : ((tid >> 4) + 16 * (k & 1)); };
    const int chunk_c = tid & (CH - 1);
    // The RHT's random signs are applied as the tile enters LDS: a chunk is
    // one token row j of its block, so one sign bit (mask bit j) covers it.
    auto sign_word = [&](int j) -> uint32_t {
        if (!RHT) return 0u;
        const uint32_t sb = (mask >> j) & 1u;
        return BF16 ? sb * 0x80008000u : sb << 31;
    };

    // Vector path.  Per block row, each thread resolves the row of x behind
    // each of its chunks once (a valid row where the chunk holds no token)
    // and keeps one bit per chunk, set where it holds a token; the column
    // tiles of that block row then cost one address per chunk.
    int32_t xr[NLD];
    uint32_t keep = 0;
    auto rows_for = [&](int64_t pb0) {
        int64_t t0;
        int32_t n;
        block_info(pb0, t0, n);
        keep = 0;
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int b = chunk_b(k), j = chunk_j(k);
            const int64_t tb = bcast64(t0, b);
            const int32_t nb = __builtin_amdgcn_readlane(n, b);
            const bool ok = j < nb;
            const int64_t r = ok ? tb + j : (nb > 0 ? tb : 0);   // a block past the end: position 0
            xr[k] = ridx ? ridx[r] : (int32_t)r;
            keep |= (ok ? 1u : 0u) << k;
        }
    };
    // one row of x spans at most 4 GiB - 1 bytes (checked by the host)
    const uint32_t rowbytes = (uint32_t)cols * (uint32_t)TL::EB;
    auto load_regs = [&](uint4* v, uint32_t& kb, int64_t c0) {
        int64_t col = c0 + chunk_c * (16 / TL::EB);
        const bool cok = col < cols;
        kb = cok ? keep : 0u;
        if (!cok) col = 0;                                  // loaded, then zeroed
        const uint8_t* base = (const uint8_t*)x + col * TL::EB;
#pragma unroll
        for (int k = 0; k < NLD; ++k) v[k] = *(const uint4*)(base + (uint64_t)(uint32_t)xr[k] * rowbytes);
    };
    // into LDS: chunks without a token become zeros, then the sign applies
    // (a zero with its sign flipped is -0, as in the scalar path)
    auto store_regs = [&](const uint4* v, uint32_t kb) {
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)kb, k, 1);   // all ones or zero
            const uint32_t sg = sign_word(chunk_j(k));
            const uint4 w = make_uint4((v[k].x & m) ^ sg, (v[k].y & m) ^ sg, (v[k].z & m) ^ sg, (v[k].w & m) ^ sg);
            *(uint4*)(tile + chunk_b(k) * TL::BSTRIDE + chunk_j(k) * TL::ROWB + chunk_c * 16) = w;
        }
    };

    // Tiles run block-row-major; workgroup w takes the contiguous range
    // [w T / G, (w + 1) T / G) of the T tiles that hold data, so its tiles
    // share block rows (and their source rows) and every workgroup gets the
    // same count within one.
    const int64_t brows = (nblk_total + CT_BLOCKS - 1) / CT_BLOCKS;
    const int64_t ntiles = brows * col_tiles;
    const int64_t tbeg = ntiles * blockIdx.x / gridDim.x, tend = ntiles * (blockIdx.x + 1) / gridDim.x;
    int64_t br = tbeg / col_tiles, ct = tbeg % col_tiles;
    uint4 pre[NLD];
    uint32_t pkb = 0;
    int32_t splace = 0;          // staged scales: this lane's block placement (lanes 0..7)
    int64_t rq_tb = 0;           // ROWQ: first grouped row of this thread's block, its
    int32_t rq_nb = 0;           //       token count, and the block row they are for
    int64_t rq_br = -1;
    int64_t splace_br = -1;      // the block row it was computed for
    if (vec && tbeg < tend) {
        rows_for(br * CT_BLOCKS);
        load_regs(pre, pkb, ct * CT_COLS);
    }
    for (int64_t tl = tbeg; tl < tend; ++tl) {
        const int64_t pb0 = br * CT_BLOCKS;
        const int64_t c0 = ct * CT_COLS;
        // staged scales: lane b < 8 of every wave places block pb0 + b
        // (stage << 3 | slot; the last group starting at or before it),
        // once per block row (its column tiles share it)
        if (staged && br != splace_br) {
            splace_br = br;
            splace = 0;
            if (lane < CT_BLOCKS && pb0 + lane < nblk_total) {
                const int64_t pb = pb0 + lane;
                int lo = 0, hi = num_groups - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (pstart[mid] <= pb) lo = mid; else hi = mid - 1;
                }
                const int32_t rel = (int32_t)(pb - pstart[lo]);
                splace = ((sstart[lo] + (rel >> 3)) << 3) | (rel & 7);
            }
        }

        // ---- the tile into LDS (rows past a group's end, columns past cols: 0)
        if (vec) {
            store_regs(pre, pkb);
        } else {
            int64_t t0;
            int32_t n;
            block_info(pb0, t0, n);
            for (int k = 0; k < CT_BLOCKS * 32 * CT_COLS / 256; ++k) {
                const int b = k >> 3, j = (tid >> 6) + 4 * (k & 7), cc = tid & 63;
                const int64_t tb = bcast64(t0, b);
                const int32_t nb = __builtin_amdgcn_readlane(n, b);
                const int64_t col = c0 + cc;
                uint8_t* dst = tile + b * TL::BSTRIDE + j * TL::ROWB + cc * TL::EB;
                const bool ok = j < nb && col < cols;
                const int64_t src = ok ? ((ridx ? (int64_t)ridx[tb + j] : tb + j) * cols + col) : 0;
                const uint32_t sg = sign_word(j);
                if (BF16) *(uint16_t*)dst = (uint16_t)((ok ? ((const uint16_t*)x)[src] : 0u) ^ (sg & 0xFFFFu));
                else *(uint32_t*)dst = (ok ? ((const uint32_t*)x)[src] : 0u) ^ sg;
            }
        }
        __syncthreads();
        // ---- the next tile (of this or the next block row) into registers
        // while this one is quantized
        const bool wrap = ct + 1 == col_tiles;
        const int64_t nbr = wrap ? br + 1 : br, nct = wrap ? 0 : ct + 1;
        if (vec && tl + 1 < tend) {
            if (wrap) rows_for(nbr * CT_BLOCKS);
            load_regs(pre, pkb, nct * CT_COLS);
        }

        // ---- ROWQ: the row-wise quantization of the tile's tokens.  Thread t
        // takes token row t % 32 of block t / 32 and both 32-column blocks of
        // it; rows past a group's end (padding) have no row-wise counterpart.
        // The RHT's signs, applied as the tile entered LDS, are undone.
        if (ROWQ) {
            const int rb = tid >> 5, rj = tid & 31;
            if (br != rq_br) {
                // once per block row (its column tiles share it): block rb's
                // first grouped row and its token count
                rq_br = br;
                int64_t t0;
                int32_t n;
                block_info(pb0, t0, n);                  // lane b < 8 of each wave: block b
                rq_tb = (int64_t)(((uint64_t)(uint32_t)__shfl((int)((uint64_t)t0 >> 32), rb) << 32) |
                                  (uint32_t)__shfl((int)(uint32_t)t0, rb));
                rq_nb = __shfl(n, rb);
            }
            const int32_t nb = rq_nb;
            const int64_t prow = rq_tb + rj;             // the token's grouped row
            // The RHT's signs, flipped on the way into LDS, are undone on the
            // codes: rounding is symmetric, so the codes of -x are those of x
            // with every nibble's sign bit flipped (zeros included), and the
            // block amax does not see signs.
            const uint32_t cflip = sign_word(rj) ? 0x88888888u : 0u;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int64_t c = c0 + 32 * half;
                if (rj < nb && c < cols) {
                    const uint8_t* src = tile + rb * TL::BSTRIDE + rj * TL::ROWB + half * 32 * TL::EB;
                    float v[32];
                    if (BF16) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint4 w = *(const uint4*)(src + 16 * k);
                            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                v[8 * k + 2 * e] = bf16lo(ww[e]);
                                v[8 * k + 2 * e + 1] = bf16hi(ww[e]);
                            }
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const uint4 w = *(const uint4*)(src + 16 * k);
                            v[4 * k + 0] = __uint_as_float(w.x); v[4 * k + 1] = __uint_as_float(w.y);
                            v[4 * k + 2] = __uint_as_float(w.z); v[4 * k + 3] = __uint_as_float(w.w);
                        }
                    }
                    uint32_t am = 0;
#pragma unroll
                    for (int e = 0; e < 32; ++e) am = max(am, __float_as_uint(v[e]) & 0x7FFFFFFFu);
                    const uint32_t byte = scale_byte_from_amax_bits(am);
                    const float sc = scale_operand(byte);
                    uint32_t w4[4];
                    // counter of elements 8 qq .. 8 qq + 7 of the block: (ebase + 8 qq) / 8
                    const uint64_t e8 = (a.row_index_base + (uint64_t)prow * (uint64_t)cols + (uint64_t)c) >> 3;
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        if (ROWQ == 2) {
                            const uint64_t g8 = e8 + (uint64_t)qq;
                            const u32x4 r = philox4x32_10((uint32_t)g8, (uint32_t)(g8 >> 32), a.row_stream_id, 0u,
                                                          k0, k1);
                            w4[qq] = cvt8_sr(v + 8 * qq, sc, r);
                        } else {
                            w4[qq] = cvt8_rne(v + 8 * qq, sc);
                        }
                        w4[qq] ^= cflip;
                    }
                    if (byte == 0xFFu) w4[0] = w4[1] = w4[2] = w4[3] = 0;
                    *(uint4*)(a.row_codes + prow * a.row_ld + (c >> 5) * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                    const uint32_t rcb = (uint32_t)(c >> 5);
                    if (a.row_srows)
                        a.row_scales[((rcb >> 3) * a.row_srows + (uint32_t)prow) * 8u + (rcb & 7u)] = (uint8_t)byte;
                    else
                        a.row_scales[prow * (cols >> 5) + (c >> 5)] = (uint8_t)byte;
                }
            }
        }

        // ---- quantize: thread = (block b, column pair cp), one column at a time
        const int b = tid >> 5, cp = tid & 31;
        uint4 outc[2];
        uint32_t outs[2];
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            float t[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint8_t* src = tile + b * TL::BSTRIDE + j * TL::ROWB + (cp * 2 + side) * TL::EB;
                if (BF16) t[j] = __uint_as_float((uint32_t)(*(const uint16_t*)src) << 16);
                else t[j] = *(const float*)src;
            }
            const int64_t c = c0 + 2 * cp + side;
            uint32_t am = 0;
            if (RHT) {
                // the signs are already in t (applied on the way into LDS).
                // The block amax comes from the last butterfly stage's
                // inputs: the larger of |a + b| and |a - b| is fl(|a| + |b|)
                // (rounding is monotonic and symmetric), a NaN input gives a
                // NaN sum, and the scaling by c32 preserves the maximum.
                fwht_inlane<32, 16>(t);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float a = t[j], bb = t[j + 16];
                    am = max(am, __float_as_uint(fabsf(a) + fabsf(bb)));
                    t[j] = a + bb;
                    t[j + 16] = a - bb;
                }
                const float cc = __uint_as_float(0x3E3504F3u);
                am = __float_as_uint(__uint_as_float(am) * cc) & 0x7FFFFFFFu;
#pragma unroll
                for (int j = 0; j < 32; ++j) t[j] = t[j] * cc;
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) am = max(am, __float_as_uint(t[j]) & 0x7FFFFFFFu);
            }
            const uint32_t byte = scale_byte_from_amax_bits(am);
            const float sc = scale_operand(byte);
            uint32_t w[4];
            // counter of elements 8 qq .. 8 qq + 7: (ebase + 8 qq) / 8 = ebase / 8 + qq
            const uint64_t e8 = (index_base + (uint64_t)c * (uint64_t)kp + (uint64_t)(pb0 + b) * 32) >> 3;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                if (SR) {
                    const uint64_t g8 = e8 + (uint64_t)qq;
                    const u32x4 r = philox4x32_10((uint32_t)g8, (uint32_t)(g8 >> 32), stream_id, 0u, k0, k1);
                    w[qq] = cvt8_sr(t + 8 * qq, sc, r);
                } else {
                    w[qq] = cvt8_rne(t + 8 * qq, sc);
                }
            }
            if (byte == 0xFFu) w[0] = w[1] = w[2] = w[3] = 0;   // non-finite block: codes are 0
            outc[side] = make_uint4(w[0], w[1], w[2], w[3]);
            outs[side] = byte;
        }
        __syncthreads();                                     // every thread is done reading the tile
        // ---- regroup: column-major codes [64][8 x 16 B], then scales [64][8]
        uint8_t* oc = tile;
        uint8_t* os = tile + CT_COLS * CT_OUT_PITCH;
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int col = 2 * cp + side;
            *(uint4*)(oc + col * CT_OUT_PITCH + b * 16) = outc[side];
            os[col * CT_BLOCKS + b] = (uint8_t)outs[side];
        }
        __syncthreads();
        // ---- store: 8 lanes write one column's 8 blocks (128 contiguous bytes)
        const int64_t nv = min((int64_t)CT_BLOCKS, nblk_total - pb0);
        // staged: this thread's block ch = tid % 8 (the same for both k), from
        // lane ch, read with every lane active
        const int32_t pl = staged ? __shfl(splace, tid & 7) : 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = tid + 256 * k;
            const int col = q >> 3, ch = q & 7;
            if (c0 + col < cols && ch < nv) {
                *(uint4*)(codes + (c0 + col) * (kp >> 1) + (pb0 + ch) * 16) =
                    *(const uint4*)(oc + col * CT_OUT_PITCH + ch * 16);
                int64_t si = (c0 + col) * kp_blocks + pb0 + ch;
                // (the host keeps the staged array below 4 GiB: 32-bit offsets)
                if (staged) si = (uint32_t)(((uint32_t)(pl >> 3) * (uint32_t)cols + (uint32_t)(c0 + col)) * 8u +
                                            (uint32_t)(pl & 7));
                scales[si] = os[col * CT_BLOCKS + ch];
            }
        }
        __syncthreads();                                     // LDS is reused by the next tile
        br = nbr;
        ct = nct;
    }
}

// ===========================================================================
// 32x32 quantization (RTNE), both layouts in one pass.
// A workgroup owns a super-strip of up to 8 tile rows x 8 tiles (256 x 256
// elements) and walks its tile rows one at a time.  Per tile row, thread t
// takes row r = t / 8 of tile j = t % 8 (32 contiguous elements); the tile
// amax is reduced across lanes and waves, the row's 16 code bytes go straight
// to the as-given layout (8 threads cover a row's 128 contiguous bytes), and
// are kept in LDS.  After the last tile row the codes are regrouped by
// column, so every column of W leaves as up to 128 contiguous bytes of the
// transposed layout written by one workgroup (full lines, no partial lines
// merged across XCDs).
// ===========================================================================
constexpr int Q2_TR = 8;   // tile rows per super-strip

// Transpose an 8 x 8 matrix of 4-bit codes held as 8 words, element (r, c) in
// nibble c of a[r]: afterwards element (r, c) is nibble r of a[c].  Three
// rounds swap the off-diagonal 4x4, 2x2 and 1x1 blocks.
__device__ __forceinline__ void transpose_nibbles_8x8(uint32_t* a) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t t = ((a[r] >> 16) ^ a[r + 4]) & 0x0000FFFFu;
        a[r] ^= t << 16;
        a[r + 4] ^= t;
    }
    constexpr int rows2[4] = {0, 1, 4, 5};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rows2[i];
        const uint32_t t = ((a[r] >> 8) ^ a[r + 2]) & 0x00FF00FFu;
        a[r] ^= t << 8;
        a[r + 2] ^= t;
    }
#pragma unroll
    for (int r = 0; r < 8; r += 2) {
        const uint32_t t = ((a[r] >> 4) ^ a[r + 1]) & 0x0F0F0F0Fu;
        a[r] ^= t << 4;
        a[r + 1] ^= t;
    }
}

// De-oscillation (DEOSC): a hysteresis band against the previous step's
// codes.  While a tile's scale byte equals the previous one (neither 0xFF),
// an element whose round-to-nearest-even code differs from its previous code
// c keeps c while its scaled magnitude A = |w| / 2^X lies strictly inside
// (lo[m], hi[m]), m = c & 7, and its sign is c's (any sign when m = 0):
// the rounding interval of level m widened by f - 1/2 of a grid step on
// each side, f = 1/2 + margin / 64 (lo[0] = -inf, hi[7] = +inf).  This is
// the signed-grid band (q - f (q - q_dn), q + f (q_up - q)) of the previous
// value q, written on magnitudes.  Every bound is a multiple of 2^-7, exact
// in fp32, and A is exact (a power-of-two scaling), so each decision is
// exact.
struct DeoscArgs {
    const uint8_t* prev_codes;   // as-given layout of the previous call (may alias codes)
    int64_t prev_ld;
    const uint8_t* prev_scales;  // [batch x rows/32 x cols/32] (may alias scales)
    float f;                     // 1/2 + margin / 64
    float scale_keep;            // 4 - margin / 16: a one-binade drop of the tile amax above
                                 // scale_keep * 2^X_prev keeps the previous scale byte
    uint16_t* flips;             // per tile: elements whose decoded value changed (may be NULL)
};

// Decoded E2M1 value as (mantissa bit, exponent) for magnitude code m >= 1:
// GRID[m] = (1 + mant / 2) 2^e.  Two nonzero codes under scale bytes s, t
// decode to the same value iff their signs, mantissa bits and e + s agree.
__device__ __forceinline__ uint32_t e2m1_value_key(uint32_t m, uint32_t sbyte) {
    const uint32_t mant = m > 1u ? (m & 1u) : 0u;
    return (mant << 16) | ((m >> 1) + sbyte);      // e + 1 + s, never negative
}

template <bool BF16, bool DEOSC>
__global__ __launch_bounds__(256) void q2d_kernel(const void* __restrict__ w, int64_t rows, int64_t cols,
                                                  int64_t col_strips, int64_t row_strips, int64_t nsuper,
                                                  uint8_t* __restrict__ codes, int64_t ld,
                                                  uint8_t* __restrict__ scales,
                                                  uint8_t* __restrict__ codes_t, int64_t ld_t,
                                                  uint8_t* __restrict__ scales_t, DeoscArgs dz) {
    __shared__ uint32_t wave_amax[Q2_TR][4][8];    // per tile row: each wave's maximum per tile
    __shared__ uint8_t tile_scale[Q2_TR][8];
    __shared__ float2 band[8];                      // DEOSC: (lo, hi) per previous magnitude code
    __shared__ uint32_t wave_flips[Q2_TR][4][8];    // DEOSC: flips per tile row, wave and tile
    if (DEOSC && threadIdx.x < 8) {
        const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
        const int m = threadIdx.x;
        const float lo = m == 0 ? -__builtin_inff() : grid[m] - dz.f * (grid[m] - grid[m - 1]);
        const float hi = m == 7 ? __builtin_inff() : grid[m] + dz.f * (grid[m + 1] - grid[m]);
        band[m] = make_float2(lo, hi);
    }
    if (DEOSC) __syncthreads();
    // [tile row][tile][row] 16 bytes of row codes; each tile row padded by one
    // entry so the 8 tile rows of one tile fall in different LDS banks
    constexpr int TC_TS = 8 * 32 + 1;
    __shared__ uint4 tcodes[Q2_TR * TC_TS];
    const int t = threadIdx.x;
    const int r = t >> 3;          // 0..31
    const int j = t & 7;           // tile within the strip
    const int lane = t & 63;
    const int wv = t >> 6;
    const int64_t tiles_per_row = cols >> 5;
    const int64_t row_tiles = rows >> 5;
    for (int64_t s = blockIdx.x; s < nsuper; s += gridDim.x) {
        const int64_t bt = s / (row_strips * col_strips);
        const int64_t rem = s - bt * row_strips * col_strips;
        const int64_t rs = rem / col_strips;
        const int64_t cs = rem - rs * col_strips;
        const int64_t tr0 = rs * Q2_TR;
        const int ntr = (int)min((int64_t)Q2_TR, row_tiles - tr0);
        const int64_t tile = cs * 8 + j;
        const bool valid = tile < tiles_per_row;
        // this thread's 32 elements of tile row ts, as raw words; the next
        // tile row's are loaded before this one's block-wide amax reduction
        constexpr int NQ = BF16 ? 4 : 8;
        uint4 raw[NQ];
        auto load_raw = [&](int ts) {
            const int64_t grow = bt * rows + (tr0 + ts) * 32 + r;
            const uint4* p = (const uint4*)((const uint8_t*)w + (grow * cols + tile * 32) * (BF16 ? 2 : 4));
#pragma unroll
            for (int k = 0; k < NQ; ++k) raw[k] = valid ? p[k] : make_uint4(0, 0, 0, 0);
        };
        load_raw(0);
        for (int ts = 0; ts < ntr; ++ts) {
            const int64_t tr = tr0 + ts;
            const int64_t grow = bt * rows + tr * 32 + r;      // global row in the batch stack
            float v[32];
#pragma unroll
            for (int k = 0; k < NQ; ++k) {
                const uint4 q = raw[k];
                if (BF16) {
                    v[8 * k + 0] = bf16lo(q.x); v[8 * k + 1] = bf16hi(q.x);
                    v[8 * k + 2] = bf16lo(q.y); v[8 * k + 3] = bf16hi(q.y);
                    v[8 * k + 4] = bf16lo(q.z); v[8 * k + 5] = bf16hi(q.z);
                    v[8 * k + 6] = bf16lo(q.w); v[8 * k + 7] = bf16hi(q.w);
                } else {
                    v[4 * k + 0] = __uint_as_float(q.x); v[4 * k + 1] = __uint_as_float(q.y);
                    v[4 * k + 2] = __uint_as_float(q.z); v[4 * k + 3] = __uint_as_float(q.w);
                }
            }
            if (ts + 1 < ntr) load_raw(ts + 1);
            // DEOSC: this row's previous codes and the tile's previous scale,
            // read before the new ones are written (the block-wide barriers
            // below separate every thread's read from the scale's write)
            uint4 pcw = make_uint4(0, 0, 0, 0);
            uint32_t pbyte = 0xFFu;
            if (DEOSC && valid) {
                pcw = *(const uint4*)(dz.prev_codes + grow * dz.prev_ld + tile * 16);
                pbyte = dz.prev_scales[(bt * row_tiles + tr) * tiles_per_row + tile];
            }
            uint32_t am = 0;
#pragma unroll
            for (int k = 0; k < 32; ++k) am = max(am, __float_as_uint(v[k]) & 0x7FFFFFFFu);
            // lanes with the same j within the wave: xor 8, 16, 32
            am = max(am, (uint32_t)__shfl_xor((int)am, 8));
            am = max(am, (uint32_t)__shfl_xor((int)am, 16));
            am = max(am, (uint32_t)__shfl_xor((int)am, 32));
            if (lane < 8) wave_amax[ts][wv][lane] = am;
            __syncthreads();
            // Every thread forms its tile's scale from the four waves' maxima.
            // Each tile row has its own slots, so no wave overwrites maxima
            // another is still reading: one barrier per tile row.
            const uint32_t m = max(max(wave_amax[ts][0][j], wave_amax[ts][1][j]),
                                   max(wave_amax[ts][2][j], wave_amax[ts][3][j]));
            uint32_t byte = scale_byte_from_amax_bits(m);
            // DEOSC: an amax that dropped just below the previous scale's
            // range (the rule one byte below the previous byte p, amax >=
            // (4 - margin / 16) 2^(p - 127)) keeps p; every element then fits
            // without clipping
            if (DEOSC && valid && pbyte != 0xFFu && byte != 0xFFu && byte + 1u == pbyte &&
                __uint_as_float(m) >= dz.scale_keep * __uint_as_float(pbyte << 23))
                byte = pbyte;
            if (t < 8) tile_scale[ts][t] = (uint8_t)byte;      // (r = 0, j = t) for the transposed scales
            const float sc = scale_operand(byte);
            // non-finite tile: codes are 0 (a mask, so the four converts stay
            // branch-free and the row's 16 code bytes go out as one store)
            const uint32_t keep = byte == 0xFFu ? 0u : 0xFFFFFFFFu;
            uint32_t cw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) cw[k] = cvt8_rne(v + 8 * k, sc) & keep;
            if (DEOSC) {
                const bool hyst = byte == pbyte && byte != 0xFFu;
                const bool nan_tile = byte == 0xFFu || pbyte == 0xFFu;
                const float inv = __uint_as_float((254u - byte) << 23);   // 2^-X (byte <= 252 for finite w)
                const uint32_t pw[4] = {pcw.x, pcw.y, pcw.z, pcw.w};
                uint32_t nflip = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t out = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = v[8 * k + e];
                        const uint32_t cr = (cw[k] >> (4 * e)) & 0xFu, cp = (pw[k] >> (4 * e)) & 0xFu;
                        const uint32_t m = cp & 7u;
                        const float A = fabsf(x) * inv;
                        const float2 b = band[m];
                        const bool side = m == 0u || (cp >> 3) == (__float_as_uint(x) >> 31);
                        const uint32_t c = (hyst && side && A > b.x && A < b.y) ? cp : cr;
                        out |= c << (4 * e);
                        const uint32_t mn = c & 7u;
                        const bool differ = (mn == 0u) != (m == 0u) ||
                                            (mn != 0u && ((c ^ cp) >> 3 || e2m1_value_key(mn, byte) !=
                                                                               e2m1_value_key(m, pbyte)));
                        nflip += (nan_tile || differ) ? 1u : 0u;
                    }
                    cw[k] = out;
                }
                if (!valid) nflip = 0;
                // the tile's count: lanes with the same j (xor 8, 16, 32), then
                // across the waves after the last tile row
                nflip += (uint32_t)__shfl_xor((int)nflip, 8);
                nflip += (uint32_t)__shfl_xor((int)nflip, 16);
                nflip += (uint32_t)__shfl_xor((int)nflip, 32);
                if (lane < 8) wave_flips[ts][wv][lane] = nflip;
            }
            if (valid && codes)
                store_b128(codes + grow * ld + tile * 16, make_uint4(cw[0], cw[1], cw[2], cw[3]));
            if (valid && r == 0 && scales) scales[(bt * row_tiles + tr) * tiles_per_row + tile] = (uint8_t)byte;
            tcodes[ts * TC_TS + j * 32 + r] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        }
        __syncthreads();
        if (DEOSC && dz.flips && t < 64) {
            const int jt = t >> 3, ts = t & 7;
            const int64_t tile3 = cs * 8 + jt;
            if (tile3 < tiles_per_row && ts < ntr)
                dz.flips[(bt * row_tiles + tr0 + ts) * tiles_per_row + tile3] =
                    (uint16_t)(wave_flips[ts][0][jt] + wave_flips[ts][1][jt] + wave_flips[ts][2][jt] +
                               wave_flips[ts][3][jt]);
        }
        if (codes_t) {
            // thread t: tile row ts = t % 8, code word w = (t / 8) % 4 (columns
            // 8w .. 8w+7) of tile jj = t / 32.  It reads that word of the
            // tile's 32 rows, transposes four 8 x 8 nibble blocks, and writes
            // the 8 columns' 16-byte runs; the 8 threads of one (tile, word)
            // cover tile rows 0..7, i.e. 128 contiguous bytes per column.
            const int ts = t & 7, w = (t >> 3) & 3, jj = t >> 5;
            const int64_t tile2 = cs * 8 + jj;
            if (tile2 < tiles_per_row && ts < ntr) {
                const uint32_t* src = (const uint32_t*)&tcodes[ts * TC_TS + jj * 32] + w;
                uint32_t out[8][4];             // [column 8w + c][rows 8 rb .. 8 rb + 7]
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    uint32_t a[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) a[r] = src[(rb * 8 + r) * 4];
                    transpose_nibbles_8x8(a);
#pragma unroll
                    for (int c = 0; c < 8; ++c) out[c][rb] = a[c];
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int64_t col = tile2 * 32 + 8 * w + c;
                    store_b128(codes_t + (bt * cols + col) * ld_t + (tr0 + ts) * 16,
                               make_uint4(out[c][0], out[c][1], out[c][2], out[c][3]));
                }
            }
            // transposed scales: lanes 8 jj .. 8 jj + 7 write one tile column's
            // consecutive tile-row bytes
            if (scales_t && t < 64) {
                const int jt = t >> 3, ts = t & 7;
                const int64_t tile3 = cs * 8 + jt;
                if (tile3 < tiles_per_row && ts < ntr)
                    scales_t[(bt * tiles_per_row + tile3) * row_tiles + tr0 + ts] = tile_scale[ts][jt];
            }
        }
        __syncthreads();                       // LDS is reused by the next super-strip
    }
}

// ===========================================================================
// Dequantize: a lane decodes 8 elements (one dword of codes).
// ===========================================================================
template <bool OUT_BF16, int BLOCK_ROWS>
__global__ __launch_bounds__(256) void deq_kernel(const uint8_t* __restrict__ codes, int64_t ld,
                                                  const uint8_t* __restrict__ scales,
                                                  int64_t rows, int64_t cols, int64_t nunits,
                                                  void* __restrict__ y) {
    const int64_t units_per_row = cols >> 3;
    const int64_t srows = rows / BLOCK_ROWS;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nunits;
         u += (int64_t)gridDim.x * blockDim.x) {
        const int64_t grow = u / units_per_row;                 // global row over the batch
        const int64_t cu = u - grow * units_per_row;
        const int64_t bt = grow / rows;
        const int64_t r = grow - bt * rows;
        const uint32_t cw = *(const uint32_t*)(codes + grow * ld + cu * 4);
        const uint8_t sb = scales[(bt * srows + r / BLOCK_ROWS) * (cols >> 5) + (cu >> 2)];
        const float sc = scale_operand(sb);
        float f[8];
        decode8(cw, sc, f);
        if (sb == 0xFF) {
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = __uint_as_float(0x7FC00000u);
        }
        if (OUT_BF16) {
            // every decoded value is exact in bf16: the high half is the value
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = (__float_as_uint(f[2 * k]) >> 16) | (__float_as_uint(f[2 * k + 1]) & 0xFFFF0000u);
            *((uint4*)y + u) = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
            uint4* p = (uint4*)y + 2 * u;
            p[0] = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
            p[1] = make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7]));
        }
    }
}

// ===========================================================================
// Study variants of the row-wise quantizer (outlier clipping, macro-block
// scaling).  Off the hot path: simple quad-per-block kernels.
//   macro pass: one wave per macro-block of BM elements of a row; its quads
//     walk the macro-block's 32-blocks 16 at a time (the RHT in registers
//     when on), the wave reduces |max|, and r = fl32(6 / amax) (1 when the
//     amax is 0 or not finite, or the quotient is not finite).
//   quantize: a quad per 32-block; y' = fl32(y * r), block scale for
//     fl32(rho * amax(y')), RTNE or SR as in the row quantizer.
//   decode: a lane per 8 elements, deq / r rounded once.
// ===========================================================================
template <bool BF16, bool RHT>
__device__ __forceinline__ void load_block_quad(const void* __restrict__ x, int64_t blk, int q, uint32_t m8,
                                                float* t) {
    if (BF16) {
        const uint4 w = *((const uint4*)((const uint8_t*)x + blk * 64) + q);
        t[0] = bf16lo(w.x); t[1] = bf16hi(w.x); t[2] = bf16lo(w.y); t[3] = bf16hi(w.y);
        t[4] = bf16lo(w.z); t[5] = bf16hi(w.z); t[6] = bf16lo(w.w); t[7] = bf16hi(w.w);
    } else {
        const uint4* p = (const uint4*)((const uint8_t*)x + blk * 128) + 2 * q;
        const uint4 a = p[0], b = p[1];
        t[0] = __uint_as_float(a.x); t[1] = __uint_as_float(a.y); t[2] = __uint_as_float(a.z);
        t[3] = __uint_as_float(a.w); t[4] = __uint_as_float(b.x); t[5] = __uint_as_float(b.y);
        t[6] = __uint_as_float(b.z); t[7] = __uint_as_float(b.w);
    }
    if (RHT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = __uint_as_float(__float_as_uint(t[e]) ^ (((m8 >> e) & 1u) << 31));
        rht32_quad(t, q);
    }
}

template <bool BF16, bool RHT>
__global__ __launch_bounds__(256) void q1d_ex_macro_kernel(const void* __restrict__ x, int64_t nmacro,
                                                           int64_t mblocks, uint32_t mask,
                                                           float* __restrict__ macro_r) {
    const int lane = threadIdx.x & 63, q = lane & 3;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const uint32_t m8 = (mask >> (8 * q)) & 0xFFu;
    for (int64_t mb = wave; mb < nmacro; mb += nwaves) {
        uint32_t am = 0;                              // |max| bit pattern (NaN above Inf)
        for (int64_t k = lane >> 2; k < mblocks; k += 16) {
            float t[8];
            load_block_quad<BF16, RHT>(x, mb * mblocks + k, q, m8, t);
#pragma unroll
            for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(t[e]) & 0x7FFFFFFFu);
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, d));
        if (lane == 0) {
            float r = 1.0f;
            if (am != 0u && am < 0x7F800000u) {
                const float qt = __fdiv_rn(6.0f, __uint_as_float(am));
                if (__float_as_uint(qt) < 0x7F800000u) r = qt;
            }
            macro_r[mb] = r;
        }
    }
}

template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(256) void q1d_ex_kernel(const void* __restrict__ x, int64_t nblocks, int64_t mblocks,
                                                     uint32_t mask, uint32_t k0, uint32_t k1, uint32_t stream_id,
                                                     uint64_t index_base, float clip_ratio,
                                                     const float* __restrict__ macro_r,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int lane = threadIdx.x & 63, q = lane & 3;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const uint32_t m8 = (mask >> (8 * q)) & 0xFFu;
    for (int64_t base = wave * 16; base < nblocks; base += nwaves * 16) {
        const int64_t blk = base + (lane >> 2);
        const bool ok = blk < nblocks;
        float t[8];
        if (ok) load_block_quad<BF16, RHT>(x, blk, q, m8, t);
        else
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = 0.0f;
        if (macro_r) {
            // macro-blocks run along each row and divide it, so block blk
            // lies in macro-block blk / mblocks
            const float r = ok ? macro_r[blk / mblocks] : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = t[e] * r;
        }
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(t[e]) & 0x7FFFFFFFu);
        am = quad_max_u(am);
        uint32_t byte;
        if (clip_ratio > 0.0f) {
            // the scale for fl32(rho * amax); a NaN or Inf amax stays non-finite
            byte = scale_byte_from_amax_bits(__float_as_uint(clip_ratio * __uint_as_float(am)) & 0x7FFFFFFFu);
        } else {
            // search: X - 1 instead of X when it strictly lowers the block's
            // squared RTNE error.  Each candidate's error is summed in its own
            // units in fp64 (v = y / 2^X and the difference |v| - |q| are
            // exact there, the square too): eight elements in order per lane,
            // then the quad's four sums in lane order.  X - 1 wins iff
            // S(X - 1) < 4 S(X).
            byte = scale_byte_from_amax_bits(am);
            if (byte != 0xFFu && byte > 0u) {
                double S[2];
#pragma unroll
                for (int cand = 0; cand < 2; ++cand) {
                    const uint32_t bc = byte - cand;
                    const uint32_t cw = cvt8_rne(t, scale_operand(bc));
                    float qv[8];
                    decode8(cw, scale_operand(127u), qv);              // the RTNE grid values, unscaled
                    const double inv = __longlong_as_double((long long)(1150u - bc) << 52);   // 2^-X, X = bc - 127
                    double acc = 0.0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const double d = fabs((double)t[e] * inv) - (double)fabsf(qv[e]);
                        acc = acc + d * d;
                    }
                    const int l0 = lane & ~3;
                    const double s0 = __shfl(acc, l0), s1 = __shfl(acc, l0 + 1), s2 = __shfl(acc, l0 + 2),
                                 s3 = __shfl(acc, l0 + 3);
                    S[cand] = ((s0 + s1) + s2) + s3;
                }
                if (S[1] < 4.0 * S[0]) byte -= 1u;
            }
        }
        const float sc = scale_operand(byte);
        uint32_t packed;
        if (SR) {
            const uint64_t g = (index_base + (uint64_t)blk * 32 + (uint64_t)q * 8) >> 3;
            const u32x4 rr = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u, k0, k1);
            packed = cvt8_sr(t, sc, rr);
        } else {
            packed = cvt8_rne(t, sc);
        }
        if (byte == 0xFFu) packed = 0;
        if (ok) {
            *((uint32_t*)(codes + blk * 16) + q) = packed;
            if (q == 0) scales[blk] = (uint8_t)byte;
        }
    }
}

__global__ __launch_bounds__(256) void deq_ex_kernel(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     const float* __restrict__ macro_r, int64_t munits,
                                                     int64_t nunits, float* __restrict__ y) {
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nunits;
         u += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t cw = *(const uint32_t*)(codes + u * 4);
        const uint8_t sb = scales[u >> 2];
        float f[8];
        decode8(cw, scale_operand(sb), f);
        const float r = macro_r ? macro_r[u / munits] : 1.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = sb == 0xFF ? __uint_as_float(0x7FC00000u) : __fdiv_rn(f[k], r);
        uint4* p = (uint4*)y + 2 * u;
        p[0] = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
        p[1] = make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7]));
    }
}

// ===========================================================================
// Host side
// ===========================================================================
namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workgroups that fit on the current device at `per_cu` per compute unit.
inline int resident_blocks(int per_cu) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return cus * per_cu;
}

inline int grid_for(int64_t work_items, int items_per_block) {
    int64_t g = (work_items + items_per_block - 1) / items_per_block;
    const int64_t cap = 256 * 32;   // enough resident waves; loops cover the rest
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (int)g;
}

inline mx_status launched() {
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

uint32_t host_philox_word0(uint32_t k0, uint32_t k1) {
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// Column-wise launch: persistent grid sized to residency (the bf16 RHT+SR
// variant needs ~150 VGPRs, 3 workgroups per CU; fp32 tiles take 66 KiB of
// LDS and up to ~240 VGPRs, 2 per CU).  Fills a.col_tiles and a.vec.
template <bool B, bool R, bool S, int Q>
mx_status launch_col_t(ColArgs a, hipStream_t s) {
    a.col_tiles = (a.cols + CT_COLS - 1) / CT_COLS;
    const int64_t tiles = a.col_tiles * ((a.kp / 32 + CT_BLOCKS - 1) / CT_BLOCKS);
    const int grid = (int)min(tiles, (int64_t)resident_blocks(B ? 3 : 2));
    a.vec = (a.cols % (B ? 8 : 4)) == 0;
    const size_t lds = (size_t)ColTile<B>::TILE + 4 * (size_t)(a.num_groups + 1) * (a.staged ? 2 : 1);
    if (!B) {
        // fp32 tiles take more than 64 KiB of dynamic LDS: raise the limit of
        // the instantiation about to run, on the current device, every call
        // (the library keeps no state)
        if (hipFuncSetAttribute((const void*)q1d_col_kernel<B, R, S, Q>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess) {
            (void)hipGetLastError();
            return MX_ERR_LAUNCH;
        }
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL((q1d_col_kernel<B, R, S, Q>), dim3(grid), dim3(256), lds, s, a);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <bool B, bool R, bool S>
mx_status launch_col_q(const ColArgs& a, int rowq, hipStream_t s) {
    if (rowq == 0) return launch_col_t<B, R, S, 0>(a, s);
    if (rowq == 1) return launch_col_t<B, R, S, 1>(a, s);
    return launch_col_t<B, R, S, 2>(a, s);
}

mx_status launch_col(const ColArgs& a, bool bf, bool rh, bool sr, int rowq, hipStream_t s) {
    if (bf) {
        if (rh) return sr ? launch_col_q<true, true, true>(a, rowq, s) : launch_col_q<true, true, false>(a, rowq, s);
        return sr ? launch_col_q<true, false, true>(a, rowq, s) : launch_col_q<true, false, false>(a, rowq, s);
    }
    if (rh) return sr ? launch_col_q<false, true, true>(a, rowq, s) : launch_col_q<false, true, false>(a, rowq, s);
    return sr ? launch_col_q<false, false, true>(a, rowq, s) : launch_col_q<false, false, false>(a, rowq, s);
}

}  // namespace

extern "C" {

int mx_version(void) { return 1; }

const char* mx_status_str(mx_status s) {
    switch (s) {
        case MX_OK: return "MX_OK";
        case MX_ERR_NULL: return "MX_ERR_NULL";
        case MX_ERR_SHAPE: return "MX_ERR_SHAPE";
        case MX_ERR_ALIGN: return "MX_ERR_ALIGN";
        case MX_ERR_DTYPE: return "MX_ERR_DTYPE";
        case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
        case MX_ERR_LAUNCH: return "MX_ERR_LAUNCH";
    }
    return "MX_ERR_UNKNOWN";
}

uint32_t mx_rht_sign_mask(uint64_t seed) { return host_philox_word0((uint32_t)seed, (uint32_t)(seed >> 32)); }

mx_status mx_rht(const void* x, mx_dtype xt, float* y, int64_t rows, int64_t cols, uint32_t sign_mask,
                 int inverse, mx_stream stream) {
    if (rows < 0 || cols <= 0 || cols % 32) return MX_ERR_SHAPE;
    if (xt != MX_F32 && xt != MX_BF16) return MX_ERR_DTYPE;
    if (rows == 0) return MX_OK;
    if (!x || !y) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return MX_ERR_ALIGN;
    const int64_t nblocks = rows * (cols / 32);
    const int grid = grid_for(nblocks, 4 * 16);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (xt == MX_BF16) {
        if (inverse) hipLaunchKernelGGL((rht_kernel<true, true>), dim3(grid), dim3(256), 0, s, x, nblocks, sign_mask, y);
        else hipLaunchKernelGGL((rht_kernel<true, false>), dim3(grid), dim3(256), 0, s, x, nblocks, sign_mask, y);
    } else {
        if (inverse) hipLaunchKernelGGL((rht_kernel<false, true>), dim3(grid), dim3(256), 0, s, x, nblocks, sign_mask, y);
        else hipLaunchKernelGGL((rht_kernel<false, false>), dim3(grid), dim3(256), 0, s, x, nblocks, sign_mask, y);
    }
    return launched();
}

#define MX_DISPATCH3_LDS(KERNEL, B, R, S, GRID, LDS, STREAM, ...)                                              \
    do {                                                                                            \
        if (B) {                                                                                    \
            if (R) {                                                                                \
                if (S) hipLaunchKernelGGL((KERNEL<true, true, true>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);   \
                else hipLaunchKernelGGL((KERNEL<true, true, false>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);    \
            } else {                                                                                \
                if (S) hipLaunchKernelGGL((KERNEL<true, false, true>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);  \
                else hipLaunchKernelGGL((KERNEL<true, false, false>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);   \
            }                                                                                       \
        } else {                                                                                    \
            if (R) {                                                                                \
                if (S) hipLaunchKernelGGL((KERNEL<false, true, true>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);  \
                else hipLaunchKernelGGL((KERNEL<false, true, false>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);   \
            } else {                                                                                \
                if (S) hipLaunchKernelGGL((KERNEL<false, false, true>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__); \
                else hipLaunchKernelGGL((KERNEL<false, false, false>), GRID, dim3(256), LDS, STREAM, __VA_ARGS__);  \
            }                                                                                       \
        }                                                                                           \
    } while (0)
#define MX_DISPATCH3(KERNEL, B, R, S, GRID, STREAM, ...) MX_DISPATCH3_LDS(KERNEL, B, R, S, GRID, 0, STREAM, __VA_ARGS__)

mx_status mx_quantize_1d(const void* x, mx_dtype xt, int64_t rows, int64_t cols, int block_axis,
                         const int32_t* group_offsets, int32_t num_groups, int64_t kp,
                         const int32_t* row_index, int use_rht,
                         uint32_t sign_mask, mx_round rnd, uint64_t seed, uint32_t stream_id,
                         uint64_t index_base, uint8_t* codes, int64_t codes_ld, uint8_t* scales,
                         mx_stream stream) {
    if (xt != MX_F32 && xt != MX_BF16) return MX_ERR_DTYPE;
    if (rnd != MX_RNE && rnd != MX_SR) return MX_ERR_UNSUPPORTED;
    if (rows < 0 || cols <= 0) return MX_ERR_SHAPE;
    if (index_base % 32) return MX_ERR_SHAPE;
    const bool bf = xt == MX_BF16, rh = use_rht != 0, sr = rnd == MX_SR;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    hipStream_t s = (hipStream_t)stream;
    const bool staged = (block_axis & MX_SCALES_STAGED) != 0;
    const bool pad256 = (block_axis & MX_GROUPS_PAD256) != 0;
    block_axis &= ~(MX_SCALES_STAGED | MX_GROUPS_PAD256);
    if (pad256 && block_axis != 0) return MX_ERR_SHAPE;
    if (block_axis == 1) {
        if (cols % 32) return MX_ERR_SHAPE;
        if (group_offsets || num_groups || kp) return MX_ERR_SHAPE;
        if (row_index) return MX_ERR_UNSUPPORTED;
        if (rows == 0) return MX_OK;
        if (!x || !codes || !scales) return MX_ERR_NULL;
        if (!aligned16(x) || !aligned16(codes)) return MX_ERR_ALIGN;
        // code row pitch: 0 = cols / 2; else at least that and a multiple of 16
        const int64_t ld = codes_ld ? codes_ld : cols / 2;
        if (ld < cols / 2 || ld % 16) return MX_ERR_SHAPE;
        if (cols / 32 > INT32_MAX) return MX_ERR_SHAPE;
        const int64_t nblocks = rows * (cols / 32);
        const int grid = grid_for(nblocks, 4 * 16 * ROW_UNROLL);
        // the grid stride in blocks: grid workgroups of 4 waves, 16 blocks per
        // wave per unrolled step
        const int64_t stride = (int64_t)grid * 4 * 16 * ROW_UNROLL;
        const int64_t bpr = cols / 32;
        // staged scales: ceil(cols / 256) stages of rows x 8 bytes, 32-bit offsets
        if (staged && (cols + 255) / 256 * rows * 8 > (int64_t)0xFFFFFFFFu) return MX_ERR_SHAPE;
        const RowPitch rp{bpr, 1.0 / (double)bpr, ld - cols / 2, ld, stride / bpr, stride % bpr,
                          staged ? (uint32_t)rows : 0u};
        (void)hipGetLastError();
        if (ld == cols / 2) {
            MX_DISPATCH3(q1d_row_kernel, bf, rh, sr, dim3(grid), s, x, nblocks, sign_mask, k0, k1, stream_id,
                         index_base, codes, scales, rp);
        } else if (bpr >= 16 * ROW_UNROLL && ld - cols / 2 < (1LL << 31)) {
            MX_DISPATCH3(q1d_row_kernel_w, bf, rh, sr, dim3(grid), s, x, nblocks, sign_mask, k0, k1, stream_id,
                         index_base, codes, scales, rp);
        } else {
            MX_DISPATCH3(q1d_row_kernel_p, bf, rh, sr, dim3(grid), s, x, nblocks, sign_mask, k0, k1, stream_id,
                         index_base, codes, scales, rp);
        }
        return launched();
    }
    if (block_axis != 0) return MX_ERR_SHAPE;
    if (num_groups < 1 || num_groups > COL_MAX_GROUPS) return MX_ERR_SHAPE;
    if (kp < 0 || kp % 32) return MX_ERR_SHAPE;
    if (codes_ld != 0 && codes_ld != kp / 2) return MX_ERR_SHAPE;   // the layout's rows are kp / 2 bytes
    if (!group_offsets) return MX_ERR_NULL;
    if (kp == 0 || rows == 0) return MX_OK;
    if (!x || !codes || !scales) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes)) return MX_ERR_ALIGN;
    if (cols > (int64_t)(0xFFFFFFFFu / (bf ? 2u : 4u))) return MX_ERR_SHAPE;   // one row of x within 4 GiB
    // staged scales: at most kp/256 + num_groups stages of cols x 8 bytes, 32-bit offsets
    if (staged && (kp / 256 + num_groups) * cols * 8 > (int64_t)0xFFFFFFFFu) return MX_ERR_SHAPE;
    ColArgs a{x, cols, group_offsets, (int)num_groups, row_index, rows, kp, 0, 0, sign_mask, k0, k1, stream_id,
              index_base, codes, scales, nullptr, 0, nullptr, 0, 0, staged ? 1 : 0, pad256 ? 8 : 1};
    return launch_col(a, bf, rh, sr, 0, s);
}

mx_status mx_quantize_1d_dual(const void* x, mx_dtype xt, int64_t rows, int64_t cols, const int32_t* group_offsets,
                              int32_t num_groups, int64_t kp, int use_rht, uint32_t sign_mask, mx_round col_rnd,
                              uint32_t col_stream_id, uint64_t col_index_base, uint8_t* col_codes,
                              uint8_t* col_scales, mx_round row_rnd, uint32_t row_stream_id,
                              uint64_t row_index_base, uint8_t* row_codes, int64_t row_codes_ld,
                              uint8_t* row_scales, uint64_t seed, int layout_flags, mx_stream stream) {
    if (xt != MX_F32 && xt != MX_BF16) return MX_ERR_DTYPE;
    if ((col_rnd != MX_RNE && col_rnd != MX_SR) || (row_rnd != MX_RNE && row_rnd != MX_SR)) return MX_ERR_UNSUPPORTED;
    if (layout_flags & ~(MX_SCALES_STAGED | MX_GROUPS_PAD256)) return MX_ERR_UNSUPPORTED;
    const bool staged = (layout_flags & MX_SCALES_STAGED) != 0;
    const bool pad256 = (layout_flags & MX_GROUPS_PAD256) != 0;
    if (rows < 0 || cols <= 0 || cols % 32) return MX_ERR_SHAPE;
    if (col_index_base % 32 || row_index_base % 32) return MX_ERR_SHAPE;
    if (num_groups < 1 || num_groups > COL_MAX_GROUPS) return MX_ERR_SHAPE;
    if (kp < 0 || kp % 32) return MX_ERR_SHAPE;
    const int64_t ld = row_codes_ld ? row_codes_ld : cols / 2;
    if (ld < cols / 2 || ld % 16) return MX_ERR_SHAPE;
    if (!group_offsets) return MX_ERR_NULL;
    if (kp == 0 || rows == 0) return MX_OK;
    if (!x || !col_codes || !col_scales || !row_codes || !row_scales) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(col_codes) || !aligned16(row_codes)) return MX_ERR_ALIGN;
    const bool bf = xt == MX_BF16;
    if (cols > (int64_t)(0xFFFFFFFFu / (bf ? 2u : 4u))) return MX_ERR_SHAPE;
    // staged scales: 32-bit offsets in both orders
    if (staged && ((kp / 256 + num_groups) * cols * 8 > (int64_t)0xFFFFFFFFu ||
                   (cols + 255) / 256 * rows * 8 > (int64_t)0xFFFFFFFFu))
        return MX_ERR_SHAPE;
    ColArgs a{x, cols, group_offsets, (int)num_groups, nullptr, rows, kp, 0, 0, sign_mask, (uint32_t)seed,
              (uint32_t)(seed >> 32), col_stream_id, col_index_base, col_codes, col_scales, row_codes, ld, row_scales,
              row_stream_id, row_index_base, staged ? 1 : 0, pad256 ? 8 : 1, staged ? (uint32_t)rows : 0u};
    return launch_col(a, bf, use_rht != 0, col_rnd == MX_SR, row_rnd == MX_SR ? 2 : 1, (hipStream_t)stream);
}

mx_status mx_quantize_1d_ex(const void* x, mx_dtype xt, int64_t rows, int64_t cols, int use_rht, uint32_t sign_mask,
                            mx_round rnd, uint64_t seed, uint32_t stream_id, uint64_t index_base, float clip_ratio,
                            int64_t macro_block, uint8_t* codes, uint8_t* scales, float* macro_r, mx_stream stream) {
    if (xt != MX_F32 && xt != MX_BF16) return MX_ERR_DTYPE;
    if (rnd != MX_RNE && rnd != MX_SR) return MX_ERR_UNSUPPORTED;
    if (rows < 0 || cols <= 0 || cols % 32 || index_base % 32) return MX_ERR_SHAPE;
    if (!(clip_ratio >= 0.0f && clip_ratio <= 1.0f)) return MX_ERR_SHAPE;
    if (macro_block < 0 || (macro_block > 0 && (macro_block % 32 || cols % macro_block))) return MX_ERR_SHAPE;
    if (rows == 0) return MX_OK;
    if (!x || !codes || !scales || (macro_block > 0 && !macro_r)) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)macro_r & 3u)) return MX_ERR_ALIGN;
    const bool bf = xt == MX_BF16, rh = use_rht != 0, sr = rnd == MX_SR;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const int64_t nblocks = rows * (cols / 32);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    int64_t mblocks = 1;
    const float* mr = nullptr;
    if (macro_block > 0) {
        mblocks = macro_block / 32;
        const int64_t nmacro = rows * (cols / macro_block);
        const int g = grid_for(nmacro, 4);
        if (bf) {
            if (rh) hipLaunchKernelGGL((q1d_ex_macro_kernel<true, true>), dim3(g), dim3(256), 0, s, x, nmacro, mblocks, sign_mask, macro_r);
            else hipLaunchKernelGGL((q1d_ex_macro_kernel<true, false>), dim3(g), dim3(256), 0, s, x, nmacro, mblocks, sign_mask, macro_r);
        } else {
            if (rh) hipLaunchKernelGGL((q1d_ex_macro_kernel<false, true>), dim3(g), dim3(256), 0, s, x, nmacro, mblocks, sign_mask, macro_r);
            else hipLaunchKernelGGL((q1d_ex_macro_kernel<false, false>), dim3(g), dim3(256), 0, s, x, nmacro, mblocks, sign_mask, macro_r);
        }
        mr = macro_r;
    }
    const int grid = grid_for(nblocks, 4 * 16);
    MX_DISPATCH3(q1d_ex_kernel, bf, rh, sr, dim3(grid), s, x, nblocks, mblocks, sign_mask, k0, k1, stream_id,
                 index_base, clip_ratio, mr, codes, scales);
    return launched();
}

mx_status mx_dequantize_1d_ex(const uint8_t* codes, const uint8_t* scales, const float* macro_r, int64_t rows,
                              int64_t cols, int64_t macro_block, float* y, mx_stream stream) {
    if (rows < 0 || cols <= 0 || cols % 32) return MX_ERR_SHAPE;
    if (macro_block < 0 || (macro_block > 0 && (macro_block % 32 || cols % macro_block))) return MX_ERR_SHAPE;
    if (rows == 0) return MX_OK;
    if (!codes || !scales || !y || (macro_block > 0 && !macro_r)) return MX_ERR_NULL;
    if (!aligned16(codes) || !aligned16(y) || ((uintptr_t)macro_r & 3u)) return MX_ERR_ALIGN;
    const int64_t nunits = rows * (cols / 8);
    const int grid = grid_for(nunits, 256);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipLaunchKernelGGL(deq_ex_kernel, dim3(grid), dim3(256), 0, s, codes, scales, macro_block > 0 ? macro_r : nullptr,
                       macro_block > 0 ? macro_block / 8 : 1, nunits, y);
    return launched();
}

mx_status mx_quantize_2d(const void* w, mx_dtype wt, int64_t batch, int64_t rows, int64_t cols, uint8_t* codes,
                         int64_t codes_ld, uint8_t* scales, uint8_t* codes_t, int64_t codes_t_ld,
                         uint8_t* scales_t, mx_stream stream) {
    if (wt != MX_F32 && wt != MX_BF16) return MX_ERR_DTYPE;
    if (batch < 0 || rows < 0 || cols < 0 || rows % 32 || cols % 32) return MX_ERR_SHAPE;
    if (batch == 0 || rows == 0 || cols == 0) return MX_OK;     // (empty tensors may have null pointers)
    if ((codes == nullptr) != (scales == nullptr)) return MX_ERR_NULL;
    if ((codes_t == nullptr) != (scales_t == nullptr)) return MX_ERR_NULL;
    if (!codes && !codes_t) return MX_ERR_NULL;
    if (!w) return MX_ERR_NULL;
    if (!aligned16(w) || (codes && !aligned16(codes)) || (codes_t && !aligned16(codes_t))) return MX_ERR_ALIGN;
    // code row pitches: 0 = contiguous rows (cols / 2, rows / 2 bytes); else
    // at least that and a multiple of 16
    const int64_t ld = codes_ld ? codes_ld : cols / 2, ld_t = codes_t_ld ? codes_t_ld : rows / 2;
    if (ld < cols / 2 || ld % 16 || ld_t < rows / 2 || ld_t % 16) return MX_ERR_SHAPE;
    const int64_t col_strips = (cols / 32 + 7) / 8;
    const int64_t row_strips = (rows / 32 + Q2_TR - 1) / Q2_TR;
    const int64_t nsuper = batch * row_strips * col_strips;
    const int grid = grid_for(nsuper, 1);
    hipStream_t s = (hipStream_t)stream;
    const DeoscArgs none{nullptr, 0, nullptr, 0.0f, 0.0f, nullptr};
    (void)hipGetLastError();
    if (wt == MX_BF16)
        hipLaunchKernelGGL((q2d_kernel<true, false>), dim3(grid), dim3(256), 0, s, w, rows, cols, col_strips,
                           row_strips, nsuper, codes, ld, scales, codes_t, ld_t, scales_t, none);
    else
        hipLaunchKernelGGL((q2d_kernel<false, false>), dim3(grid), dim3(256), 0, s, w, rows, cols, col_strips,
                           row_strips, nsuper, codes, ld, scales, codes_t, ld_t, scales_t, none);
    return launched();
}

mx_status mx_quantize_2d_deosc(const void* w, mx_dtype wt, int64_t batch, int64_t rows, int64_t cols,
                               const uint8_t* prev_codes, int64_t prev_codes_ld, const uint8_t* prev_scales,
                               int margin64, uint8_t* codes, int64_t codes_ld, uint8_t* scales, uint8_t* codes_t,
                               int64_t codes_t_ld, uint8_t* scales_t, uint16_t* flips, mx_stream stream) {
    if (wt != MX_F32 && wt != MX_BF16) return MX_ERR_DTYPE;
    if (batch < 0 || rows < 0 || cols < 0 || rows % 32 || cols % 32) return MX_ERR_SHAPE;
    if (margin64 < 0 || margin64 > 31) return MX_ERR_SHAPE;
    if (batch == 0 || rows == 0 || cols == 0) return MX_OK;     // (empty tensors may have null pointers)
    if (!w || !prev_codes || !prev_scales || !codes || !scales) return MX_ERR_NULL;
    if ((codes_t == nullptr) != (scales_t == nullptr)) return MX_ERR_NULL;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(prev_codes) || (codes_t && !aligned16(codes_t)) ||
        ((uintptr_t)flips & 1u))
        return MX_ERR_ALIGN;
    const int64_t ld = codes_ld ? codes_ld : cols / 2, ld_t = codes_t_ld ? codes_t_ld : rows / 2;
    const int64_t pld = prev_codes_ld ? prev_codes_ld : cols / 2;
    if (ld < cols / 2 || ld % 16 || ld_t < rows / 2 || ld_t % 16 || pld < cols / 2 || pld % 16) return MX_ERR_SHAPE;
    // in place: the previous codes may be the output itself, in the same layout
    if (prev_codes == codes && pld != ld) return MX_ERR_SHAPE;
    const int64_t col_strips = (cols / 32 + 7) / 8;
    const int64_t row_strips = (rows / 32 + Q2_TR - 1) / Q2_TR;
    const int64_t nsuper = batch * row_strips * col_strips;
    const int grid = grid_for(nsuper, 1);
    hipStream_t s = (hipStream_t)stream;
    const DeoscArgs dz{prev_codes, pld, prev_scales, 0.5f + (float)margin64 / 64.0f, 4.0f - (float)margin64 / 16.0f,
                       flips};
    (void)hipGetLastError();
    if (wt == MX_BF16)
        hipLaunchKernelGGL((q2d_kernel<true, true>), dim3(grid), dim3(256), 0, s, w, rows, cols, col_strips,
                           row_strips, nsuper, codes, ld, scales, codes_t, ld_t, scales_t, dz);
    else
        hipLaunchKernelGGL((q2d_kernel<false, true>), dim3(grid), dim3(256), 0, s, w, rows, cols, col_strips,
                           row_strips, nsuper, codes, ld, scales, codes_t, ld_t, scales_t, dz);
    return launched();
}

mx_status mx_dequantize(const uint8_t* codes, int64_t codes_ld, const uint8_t* scales, int64_t batch, int64_t rows,
                        int64_t cols, int block_rows, void* y, mx_dtype yt, mx_stream stream) {
    if (yt != MX_F32 && yt != MX_BF16) return MX_ERR_DTYPE;
    if (batch < 0 || rows < 0 || cols < 0 || cols % 32) return MX_ERR_SHAPE;
    if (block_rows != 1 && block_rows != 32) return MX_ERR_SHAPE;
    if (block_rows == 32 && rows % 32) return MX_ERR_SHAPE;
    if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
    if (!codes || !scales || !y) return MX_ERR_NULL;
    if (!aligned16(codes) || !aligned16(y)) return MX_ERR_ALIGN;
    const int64_t ld = codes_ld ? codes_ld : cols / 2;       // code row pitch
    if (ld < cols / 2 || ld % 16) return MX_ERR_SHAPE;
    const int64_t nunits = batch * rows * (cols / 8);
    const int grid = grid_for(nunits, 256);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (yt == MX_BF16) {
        if (block_rows == 1) hipLaunchKernelGGL((deq_kernel<true, 1>), dim3(grid), dim3(256), 0, s, codes, ld, scales, rows, cols, nunits, y);
        else hipLaunchKernelGGL((deq_kernel<true, 32>), dim3(grid), dim3(256), 0, s, codes, ld, scales, rows, cols, nunits, y);
    } else {
        if (block_rows == 1) hipLaunchKernelGGL((deq_kernel<false, 1>), dim3(grid), dim3(256), 0, s, codes, ld, scales, rows, cols, nunits, y);
        else hipLaunchKernelGGL((deq_kernel<false, 32>), dim3(grid), dim3(256), 0, s, codes, ld, scales, rows, cols, nunits, y);
    }
    return launched();
}

}  // extern "C"
