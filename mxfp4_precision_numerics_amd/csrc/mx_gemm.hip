// mx_gemm.hip -- grouped MXFP4 GEMM on the CDNA4 block-scaled FP4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E2M1, FP32 accumulation).
//
// Operand layout the MFMA reads (one wave, 32x32 output, K = 64): lane l
// supplies row (l % 32) of A and K elements [32 (l / 32), +32) as 16 bytes
// (even element in the low nibble) plus that 32-block's UE8M0 scale byte;
// B likewise per output column.  A 32-element MX block is therefore exactly
// one lane's 16-byte operand and one scale byte, so the row-major code and
// scale layouts produced by the quantizers are consumed as they are.
// Accumulator: lane l, register r holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// Tiling: a workgroup (4 waves, 2 x 2) computes a BM x BN tile of one group;
// each wave owns (BM/2) x (BN/2) as 32x32 MFMA blocks.  K advances 128 at a
// time (64 code bytes per row); A/B code tiles and their scale bytes are
// staged through double-buffered LDS with an XOR swizzle of the 16-byte
// chunks so the MFMA operand reads are bank-conflict free.
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

constexpr int BK = 128;            // K elements per stage
constexpr int BKB = BK / 2;        // code bytes per row per stage
constexpr int CHUNKS = BKB / 16;   // 16-byte chunks per row per stage (4)

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int A_CH = BM * CHUNKS / 256;   // A chunks per thread per stage
    constexpr int B_CH = BN * CHUNKS / 256;
    static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

    __shared__ uint4 lds_a[2][BM * CHUNKS];
    __shared__ uint4 lds_b[2][BN * CHUNKS];
    __shared__ uint32_t lds_as[2][BM];
    __shared__ uint32_t lds_bs[2][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---------------- tile decode ----------------
    int g = 0;
    int64_t m_begin = 0, m_end = 0, k_begin = 0, k_end = p.K;
    const int nt = (int)(blockIdx.x % (uint32_t)p.tiles_n);
    int64_t mlin = blockIdx.x / (uint32_t)p.tiles_n;
    if (p.group_dim_k == 0) {
        bool found = false;
        for (g = 0; g < p.G; ++g) {
            const int64_t gb = p.off[g], ge = p.off[g + 1];
            const int64_t mt = (ge - gb + BM - 1) / BM;
            if (mlin < mt) {
                m_begin = gb + mlin * BM;
                m_end = min(ge, m_begin + BM);
                found = true;
                break;
            }
            mlin -= mt;
        }
        if (!found) return;
    } else {
        g = (int)(mlin / p.tiles_m);
        if (g >= p.G) return;
        const int64_t mt = mlin - (int64_t)g * p.tiles_m;
        m_begin = mt * BM;
        m_end = min(p.M, m_begin + BM);
        k_begin = p.off[g];
        k_end = p.off[g + 1];
    }
    const int64_t n_begin = (int64_t)nt * BN;
    const int64_t KB = p.K / 2;      // code bytes per operand row
    const int64_t KS = p.K / 32;     // scale bytes per operand row

    const uint8_t* bcodes = p.b_codes;
    const uint8_t* bscales = p.b_scales;
    if (p.group_dim_k == 0) {
        bcodes += (int64_t)g * p.N * KB;
        bscales += (int64_t)g * (p.b_scale_2d ? (p.N / 32) * KS : p.N * KS);
    }

    // ---------------- per-thread load assignments ----------------
    // chunk id = tid + 256 * i -> tile row id / CHUNKS, chunk id % CHUNKS
    const uint8_t* a_row_ptr[A_CH];
    const uint8_t* a_srow_ptr[A_CH];
    int a_lds_idx[A_CH];
    int a_chunk[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int id = tid + 256 * i;
        const int r = id / CHUNKS, c = id % CHUNKS;
        int64_t m = m_begin + r;
        if (m >= m_end) m = m_end - 1;            // clamp: rows past the tile end are never stored
        const int64_t arow = p.a_row_index ? (int64_t)p.a_row_index[m] : m;
        a_row_ptr[i] = p.a_codes + arow * KB;
        a_srow_ptr[i] = p.a_scales + arow * KS;
        a_lds_idx[i] = r * CHUNKS + swz(r, c);
        a_chunk[i] = c;
    }
    const uint8_t* b_row_ptr[B_CH];
    const uint8_t* b_srow_ptr[B_CH];
    int b_lds_idx[B_CH];
    int b_chunk[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int id = tid + 256 * i;
        const int r = id / CHUNKS, c = id % CHUNKS;
        int64_t n = n_begin + r;
        if (n >= p.N) n = p.N - 1;
        b_row_ptr[i] = bcodes + n * KB;
        b_srow_ptr[i] = bscales + (p.b_scale_2d ? (n / 32) * KS : n * KS);
        b_lds_idx[i] = r * CHUNKS + swz(r, c);
        b_chunk[i] = c;
    }

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t klen = k_end - k_begin;
    const int nkt = (int)((klen + BK - 1) / BK);

    uint4 ra[A_CH], rb[B_CH];
    uint32_t ras[A_CH], rbs[B_CH];

    auto load_stage = [&](int kt) {
        const int64_t kbase = k_begin + (int64_t)kt * BK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int64_t k = kbase + a_chunk[i] * 32;
            if (k < k_end) {
                ra[i] = *(const uint4*)(a_row_ptr[i] + k / 2);
                ras[i] = a_srow_ptr[i][k / 32];
            } else {
                ra[i] = make_uint4(0, 0, 0, 0);
                ras[i] = 0;
            }
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int64_t k = kbase + b_chunk[i] * 32;
            if (k < k_end) {
                rb[i] = *(const uint4*)(b_row_ptr[i] + k / 2);
                rbs[i] = b_srow_ptr[i][k / 32];
            } else {
                rb[i] = make_uint4(0, 0, 0, 0);
                rbs[i] = 0;
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            lds_a[buf][a_lds_idx[i]] = ra[i];
            ((uint8_t*)lds_as[buf])[(tid + 256 * i) / CHUNKS * 4 + a_chunk[i]] = (uint8_t)ras[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            lds_b[buf][b_lds_idx[i]] = rb[i];
            ((uint8_t*)lds_bs[buf])[(tid + 256 * i) / CHUNKS * 4 + b_chunk[i]] = (uint8_t)rbs[i];
        }
    };

    if (nkt > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    const int lr = lane & 31;      // row within a 32-row MFMA block
    const int lh = lane >> 5;      // which 32-element half of K = 64

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) load_stage(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 2 + lh;
            v8i af[FM], bfr[FN];
            int as_[FM], bs_[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WM + i * 32 + lr;
                const uint4 v = lds_a[buf][r * CHUNKS + swz(r, ch)];
                af[i] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                as_[i] = ((const uint8_t*)lds_as[buf])[r * 4 + ch];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * WN + j * 32 + lr;
                const uint4 v = lds_b[buf][r * CHUNKS + swz(r, ch)];
                bfr[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                bs_[j] = ((const uint8_t*)lds_bs[buf])[r * 4 + ch];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bfr[j], acc[i][j], 4, 4, 0, as_[i], 0, bs_[j]);
        }
        if (kt + 1 < nkt) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---------------- epilogue ----------------
    const int64_t rows_here = m_end - m_begin;
    int64_t c_row0 = m_begin;
    uint8_t* cbase = (uint8_t*)p.c;
    if (p.group_dim_k == 1) cbase += (int64_t)g * p.M * p.N * (OUT_BF16 ? 2 : 4);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = n_begin + wn * WN + j * 32 + lr;
            if (col >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int rl = wm * WM + i * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
                if (rl >= rows_here) continue;
                const int64_t row = c_row0 + rl;
                const float v = acc[i][j][e] * p.alpha;
                if (OUT_BF16)
                    ((uint16_t*)cbase)[row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
                else
                    ((float*)cbase)[row * p.N + col] = v;
            }
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

    constexpr int BM = 128, BN = 128;
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
    if (tiles > 0x7FFFFFFF) return MX_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (ct == MX_BF16)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, true>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, false>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}
