// Device helpers shared by the attention kernels (k_attn.hip,
// k_attn_rows.hip): main-KV and SWA dequantisation to bf16, lane-pair
// reductions, and the LDS key-block geometry.
//
// E2M1 x E8M0 main-KV values are exact in bf16 (at most two significant
// bits times a power of two); with an E4M3 scale per 16 channels at most six
// significant bits, still exact.  gfx950's v_cvt_scalef32_pk_bf16_fp4 converts
// two E2M1 nibbles (low nibble -> low half) and multiplies by the exponent of
// its f32 scale operand.
#pragma once

#include "csa2_internal.h"

namespace csa2 {
namespace attn {

typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

// 8 E2M1 values (one dword) times `scale` -> 8 bf16 (as 4 dwords).
__device__ __forceinline__ v4i fp4x8_to_bf16(uint32_t codes, float scale) {
    auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    return v4i{__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), __builtin_bit_cast(int, c),
               __builtin_bit_cast(int, d)};
}

// The same for a scale that need not be a power of two: the conversions'
// scale operand applies only its exponent, so the values are converted to f32
// at unit scale, multiplied by the scale (exact: at most six significant bits)
// and cut to bf16 (exact for the same reason).
typedef float v2f_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int bf16_pair_mul(v2f_t f, float scale) {
    const uint32_t a = __float_as_uint(f[0] * scale), b = __float_as_uint(f[1] * scale);
    return (int)((a >> 16) | (b & 0xFFFF0000u));
}
__device__ __forceinline__ v4i fp4x8_to_bf16_mul(uint32_t codes, float scale) {
    return v4i{bf16_pair_mul(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0), scale),
               bf16_pair_mul(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1), scale),
               bf16_pair_mul(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2), scale),
               bf16_pair_mul(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3), scale)};
}

__device__ __forceinline__ float e8m0_f32(uint32_t e) { return __builtin_ldexpf(1.0f, (int)e - 127); }

// OCP E4M3 ("FN": bias 7, no infinities; the NaN codes are not allowed in a
// scale) -> f32, exactly: normal codes by their bits, subnormals m * 2^-9.
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -v : v;
}

// Main-KV scale formats: kKvMx one E8M0 per 32 channels (16 bytes a row),
// kKvE4 one E4M3 per 16 channels (32 bytes a row; the report's section 2.4.4).
enum : int { kKvMx = 0, kKvE4 = 1 };
// SWA row formats: bf16 [rows][512], or OCP MXFP8 [rows][528] (512 E4M3 codes,
// then 16 E8M0 scales, one per 32 channels)
enum : int { kSwaBf16 = 0, kSwaMx8 = 1 };

// Reductions over lane pairs l, l ^ D (D = 16 or 32) on the VALU: the swap
// leaves this lane's value and its partner's in the two results (in some order).
template <int D>
__device__ __forceinline__ v2u lane_pair(float x) {
    const uint32_t u = __float_as_uint(x);
    if constexpr (D == 16) return __builtin_amdgcn_permlane16_swap(u, u, false, false);
    else return __builtin_amdgcn_permlane32_swap(u, u, false, false);
}
template <int D>
__device__ __forceinline__ float xor_max(float x) {
    const v2u r = lane_pair<D>(x);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int D>
__device__ __forceinline__ float xor_sum(float x) {
    const v2u r = lane_pair<D>(x);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A lane's 16 query slices of a head row as bf16 MFMA operands: slice ks holds
// channels c0 = 32 ks + 8 lg .. c0 + 7 (lg = 0..3, the lane's group), read from
// bf16 at q + qr + 32 ks.  ROPE: the query is before RoPE; the channels from
// 448 on (slices 14 and 15, whatever lg) are widened to f32, rotated by the
// row's angles cs and cast back to nearest even, and every other channel goes
// through the same cast (which leaves a bf16 value as it is, except that a NaN
// gets its quiet bit set).  All loads are issued before the first is used.
template <int ROPE>
__device__ __forceinline__ void load_q16(v8bf (&Q)[16], const uint16_t* q, int64_t qr, int lg, const float* cs) {
    v4i w[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) w[ks] = ld16(q + qr + 32 * ks);
    if constexpr (ROPE) {
        v4f c[2][2];  // slices 14 and 15: pairs 4 lg .. 4 lg + 3 and 16 + 4 lg .. + 3
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float* p = cs + 32 * j + 8 * lg;
            c[j][0] = *reinterpret_cast<const v4f*>(p);
            c[j][1] = *reinterpret_cast<const v4f*>(p + 4);
        }
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            if (ks >= 14) {
                float f[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    f[2 * k] = __uint_as_float((uint32_t)w[ks][k] << 16);
                    f[2 * k + 1] = __uint_as_float((uint32_t)w[ks][k] & 0xFFFF0000u);
                }
                const v4f a = c[ks - 14][0], b = c[ks - 14][1];
                rope_pair(f[0], f[1], a[0], a[1], 1.0f);
                rope_pair(f[2], f[3], a[2], a[3], 1.0f);
                rope_pair(f[4], f[5], b[0], b[1], 1.0f);
                rope_pair(f[6], f[7], b[2], b[3], 1.0f);
#pragma unroll
                for (int k = 0; k < 4; ++k) w[ks][k] = (int)(bf16_rne(f[2 * k]) | (bf16_rne(f[2 * k + 1]) << 16));
            } else {
                // per bf16 half: its magnitude plus 0x7F carries into bit 15
                // exactly for a NaN (magnitude above 0x7F80); that bit moved to
                // bit 6 is the quiet bit (the halves cannot carry into each other)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t d = (uint32_t)w[ks][k];
                    w[ks][k] = (int)(d | ((((d & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u) >> 9));
                }
            }
        }
    }
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Q[ks] = __builtin_bit_cast(v8bf, w[ks]);
}

// Final store of output channel c of a head row (value x, this lane's; the
// partner channel c ^ 1 sits in lane l ^ 1).  ROPE: the channels from 448 on
// (rot) are turned back by their pair's angle (co, si), negated, and every
// channel is cast to bf16; the even lane of each pair stores both.  Every lane
// of the wave calls it.  The angles come in as values, loaded by the caller
// ahead of the stores, so that no store waits for a load of its own.
template <int ROPE>
__device__ __forceinline__ void store_out(void* out, int64_t off, int c, float x, bool rot, float2 cs) {
    if constexpr (ROPE) {
        // the partner lane's value by a DPP swap of adjacent lanes (quad_perm 1, 0, 3, 2)
        const float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
        if ((c & 1) == 0) {
            float a = x, b = y;
            if (rot) rope_pair(a, b, cs.x, cs.y, -1.0f);
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + off) = bf16_rne(a) | (bf16_rne(b) << 16);
        }
    } else {
        reinterpret_cast<float*>(out)[off] = x;
    }
}

// The (cos, sin) of the pairs a lane's output channels 448 + 16 j + li
// (j < 4, li = lane % 16) belong to: pair (16 j + li) / 2 of the row's angles
// cs, read at the even channel of the pair.
__device__ __forceinline__ void load_out_angles(float2 (&a)[4], const float* cs, int li) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const float2*>(cs + 16 * j + (li & ~1));
}

constexpr int KB = 64;               // keys per block
constexpr int LROW = 512 + 8;        // LDS row stride of a staged key in bf16 (16 B of padding)

}  // namespace attn
}  // namespace csa2
