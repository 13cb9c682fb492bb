// mx_device.h -- device helpers shared by the libmx355 kernels (gfx950).
//
// Numerics follow the contract stated in include/mx.h.  Everything that
// decides a code is exact or done in the contract's fp32 order:
//   * the RHT uses fp32 butterflies in the stage order 1, 2, 4, 8, 16 and one
//     multiply by c = fp32(2^-2.5); this file is compiled with
//     -ffp-contract=off so no add is fused with a multiply;
//   * the block scale comes from the exponent field of the amax (never log2);
//   * scaling by 2^-X, rounding, saturation and packing are done by the CDNA4
//     conversion instructions v_cvt_scalef32_[sr_]pk_fp4_f32, whose scale
//     operand is read as a UE8M0 exponent (fp32 bits = byte << 23) and which
//     compute RTNE(x / 2^X) (ties to even, saturating, sign of zero kept).
//     For SR each element is converted with the random word (~r16) << 16 as
//     its slot sees it: the instruction rounds the magnitude up iff its 22
//     random bits plus the 22-bit truncated fraction carry, which with the
//     low 6 random bits zero is exactly r16 < D.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Key is uniform across
// the wave in every caller, so the key schedule stays in scalar registers.
// ---------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);  // xor3
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// ---------------------------------------------------------------------------
// bf16 / fp32 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite and infinite inputs; a NaN
// stays a NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One 16-byte vector store to a 16-byte-aligned global address.  Used where
// the compiler's address strength reduction would otherwise split the store
// into four dword stores.  The trailing s_nop covers the one wait state a
// VALU write to the store's data registers needs after a 16-byte store.
__device__ __forceinline__ void store_b128(void* p, uint4 v) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v d = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" :: "v"(p), "v"(d) : "memory");
}

// ---------------------------------------------------------------------------
// Block scale from the amax bit pattern (sign already cleared):
//   exponent field E; byte = max(E - 2, 0); E == 255 (NaN/Inf) -> 0xFF.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t scale_byte_from_amax_bits(uint32_t amax_bits) {
    const uint32_t E = amax_bits >> 23;
    const uint32_t b = __builtin_elementwise_sub_sat(E, 2u);     // max(E - 2, 0)
    return E >= 255u ? 0xFFu : b;
}

// fp32 whose exponent field is the UE8M0 byte: the conversion instructions'
// scale operand.
__device__ __forceinline__ float scale_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// ---------------------------------------------------------------------------
// Conversion of 8 fp32 values (one lane's share of a block) to 8 codes
// (one dword, element e in nibble e).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t cvt8_rne(const float* v, float sc) {
    uint32_t u = 0;
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, v[0], v[1], sc, 0);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, v[2], v[3], sc, 1);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, v[4], v[5], sc, 2);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, v[6], v[7], sc, 3);
    return u;
}

// The SR conversion writes only the selected byte of its destination and
// keeps the other three, but the compiler builtin does not tie its "old"
// operand to the destination register (the other bytes then come from
// whatever register was picked).  This wrapper states the read-modify-write
// explicitly.  Register operands only; byte select J is encoded in op_sel.
template <int J>
__device__ __forceinline__ uint32_t cvt_sr_fp4_byte(uint32_t old, v2f src, uint32_t rnd, float sc) {
    if constexpr (J == 0)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(old) : "v"(src), "v"(rnd), "v"(sc));
    else if constexpr (J == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(old) : "v"(src), "v"(rnd), "v"(sc));
    else if constexpr (J == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(old) : "v"(src), "v"(rnd), "v"(sc));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(old) : "v"(src), "v"(rnd), "v"(sc));
    return old;
}

// The two random words of one Philox word w, one multiply-add each:
//   even: (0xFFFF - lo16) << 16 = lo24(w) * -2^16 + 0xFFFF0000 (mod 2^32);
//   odd:  (0xFFFF - hi16) << 15 in bits 30..15, bits 14..0 zero, from the
//         signed high half: hi16 * -2^15 + 0x7FFF8000 (mod 2^32).  Bit 31 is
//         then set for hi16 >= 2^15; the second slot sees the word shifted
//         left by one, so that bit never reaches it.
__device__ __forceinline__ uint32_t sr_word_even(uint32_t w) {
    uint32_t r;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(-65536), "v"(0xFFFF0000u));
    return r;
}
__device__ __forceinline__ uint32_t sr_word_odd(uint32_t w) {
    uint32_t r;
    asm("v_mad_i32_i16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(r) : "v"(w), "s"(-32768), "v"(0x7FFF8000u));
    return r;
}

// SR: r = the 4 Philox words for these 8 elements (element e uses word e>>1,
// low half for even e, high half for odd e).  The instruction converts a
// pair of values; its first slot rounds with the random word as given and
// its second slot with the word shifted left by one bit.  So the pair
// (v[2j], v[2j+1]) is converted twice: once with (~lo16) << 16, keeping the
// first slot's nibble (the even element), and once with ~hi16 in bits
// 30..15, which the second slot sees as (~hi16) << 16, keeping its nibble
// (the odd element).  Both words seen have their low 16 bits zero.  The two
// results are merged nibble by nibble.
__device__ __forceinline__ uint32_t cvt8_sr(const float* v, float sc, const u32x4& r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t we[4], wo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        we[j] = sr_word_even(w[j]);
        wo[j] = sr_word_odd(w[j]);
    }
    // byte 0 starts each dword: the builtin form (its destination not tied to
    // "old") leaves the other bytes unspecified, and they are written next
    uint32_t ue = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (v2f){v[0], v[1]}, we[0], sc, 0);
    uint32_t uo = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (v2f){v[0], v[1]}, wo[0], sc, 0);
    ue = cvt_sr_fp4_byte<1>(ue, (v2f){v[2], v[3]}, we[1], sc);
    uo = cvt_sr_fp4_byte<1>(uo, (v2f){v[2], v[3]}, wo[1], sc);
    ue = cvt_sr_fp4_byte<2>(ue, (v2f){v[4], v[5]}, we[2], sc);
    uo = cvt_sr_fp4_byte<2>(uo, (v2f){v[4], v[5]}, wo[2], sc);
    ue = cvt_sr_fp4_byte<3>(ue, (v2f){v[6], v[7]}, we[3], sc);
    uo = cvt_sr_fp4_byte<3>(uo, (v2f){v[6], v[7]}, wo[3], sc);
    return (ue & 0x0F0F0F0Fu) | (uo & 0xF0F0F0F0u);
}

// ---------------------------------------------------------------------------
// In-lane fp32 Walsh-Hadamard butterflies over n = 2^k values, stages
// h = 1, 2, ..., n/2 (pairs (i, i+h) -> (a+b, a-b)); HEND < n stops before
// stage HEND.
// ---------------------------------------------------------------------------
template <int N, int HEND = N>
__device__ __forceinline__ void fwht_inlane(float* t) {
#pragma unroll
    for (int h = 1; h < HEND; h <<= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if (i & h) continue;
            const float a = t[i], b = t[i + h];
            t[i] = a + b;
            t[i + h] = a - b;
        }
    }
}

// DPP quad permutations: partner lane (lane ^ 1) and (lane ^ 2) within a quad.
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t quad_xor1_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_xor2_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

// 32-point RHT butterflies + final scale for a block spread over a quad of
// lanes: lane q (= lane & 3) holds block elements 8q .. 8q+7 in t[0..7].
// Stages 1, 2, 4 run in-lane; stages 8 and 16 pair lane q with q^1 and q^2.
// A cross-lane stage computes fma(own, s, partner) = partner + s * own with
// s = +1 on the lower lane (b + a = a + b) and s = -1 on the upper lane
// (a + (-b) = a - b): one rounding each, identical to the in-order
// butterfly including the sign of an exact zero.
__device__ __forceinline__ void rht32_quad(float* t, int q) {
    fwht_inlane<8>(t);
    const float s1 = (q & 1) ? -1.0f : 1.0f;
    const float s2 = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __builtin_fmaf(t[i], s1, quad_xor1(t[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __builtin_fmaf(t[i], s2, quad_xor2(t[i]));
    const float c = __uint_as_float(0x3E3504F3u);   // fp32(2^-2.5)
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = t[i] * c;
}

// |x| bit pattern max over a quad (after the in-lane max): all 4 lanes get it.
__device__ __forceinline__ uint32_t quad_max_u(uint32_t m) {
    m = max(m, quad_xor1_u(m));
    m = max(m, quad_xor2_u(m));
    return m;
}

}  // namespace mx

namespace mx {
// Decode one dword of 8 codes with a UE8M0 scale (exact).
__device__ __forceinline__ void decode8(uint32_t cw, float sc, float* f) {
    v2f p;
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 0); f[0] = p[0]; f[1] = p[1];
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 1); f[2] = p[0]; f[3] = p[1];
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 2); f[4] = p[0]; f[5] = p[1];
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 3); f[6] = p[0]; f[7] = p[1];
}
}  // namespace mx
