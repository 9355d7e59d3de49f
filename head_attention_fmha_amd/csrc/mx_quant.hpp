// mx_quant.hpp -- OCP microscaling (MX) quantisation of the attention output
// in the kernels' epilogues (gfx950).
//
// A block of 32 consecutive head-dim columns of one output row shares an
// E8M0 scale 2^X, X = floor(log2 max|o|) - emax (emax 8 for FP8 E4M3, 2 for
// FP4 E2M1), clamped to [-127, 127] (-127 for an all-zero block).  Each
// element o / 2^X is rounded to the element format to nearest, ties to even
// (v_rndne_f32 on an exactly scaled significand), saturating at the largest
// finite magnitude (448, resp. 6).  Codes: E4M3 = sign | exponent (bias 7)
// | 3 mantissa bits, exponent field 0 for subnormals m * 2^-9; E2M1 = sign |
// exponent (bias 1) | 1 mantissa bit, exponent field 0 for 0.5.  Two E2M1
// codes share a byte, the lower column in the low nibble.  The pages'
// output-quantisation step (the FP4 pack slot of the one-way epilogue, the
// NVFP4 quantiser of the commit log at 593bc25a) is done here in the MX
// formats gfx950 implements.
#pragma once

#include "device_common.hpp"

namespace fmha {

enum OutFormat : int { kOutBf16 = 0, kOutMxFp8E4M3 = 1, kOutMxFp4E2M1 = 2 };

// floor(log2 a) for a > 0 from the exponent field (-127 for fp32 subnormals,
// which every caller clamps far above)
__device__ __forceinline__ int exponent_of(float a) { return (int)((__float_as_uint(a) >> 23) & 0xffu) - 127; }

__device__ __forceinline__ int mx_block_exp(float amax, int emax) {
    if (!(amax > 0.f)) return -127;
    return min(max(exponent_of(amax) - emax, -127), 127);
}

__device__ __forceinline__ unsigned mx_e4m3(float v) {
    const unsigned sign = (__float_as_uint(v) >> 31) << 7;
    const float a = fabsf(v);
    int e = a > 0.f ? max(exponent_of(a), -6) : -6;
    float m = rintf(ldexpf(a, 3 - e));  // significand with 3 fraction bits, or a subnormal count
    if (m >= 16.f) {                    // rounding carried into the next binade
        ++e;
        m = 8.f;
    }
    unsigned code;
    if (e > 8 || (e == 8 && m > 14.f)) code = 0x7eu;  // saturate: 448
    else if (m < 8.f) code = (unsigned)m;             // subnormal
    else code = ((unsigned)(e + 7) << 3) | ((unsigned)m - 8u);
    return sign | code;
}

__device__ __forceinline__ unsigned mx_e2m1(float v) {
    const unsigned sign = (__float_as_uint(v) >> 31) << 3;
    const float a = fabsf(v);
    int e = a > 0.f ? max(exponent_of(a), 0) : 0;
    float m = rintf(ldexpf(a, 1 - e));
    if (m >= 4.f) {
        ++e;
        m = 2.f;
    }
    unsigned code;
    if (e > 2 || (e == 2 && m > 3.f)) code = 7u;  // saturate: 6
    else if (m < 2.f) code = (unsigned)m;         // 0 or the subnormal 0.5
    else code = ((unsigned)(e + 1) << 1) | ((unsigned)m - 2u);
    return sign | code;
}

typedef short mx_short2 __attribute__((ext_vector_type(2)));

// Codes of four consecutive columns, scaled by 2^-x: FP8 -> 4 bytes, FP4 -> 2.
// While 2^x is a normal float, gfx950's scaled conversions do it in hardware
// (v_cvt_scalef32_pk_fp8_f32 / _fp4_f32: element v / 2^x, rounded to nearest
// even; FP4 saturates at 6).  The FP8 conversion gives NaN instead of
// saturating, so its inputs are first clamped to +-448 * 2^x, the largest
// finite code (448 itself, or a value that rounds to it, is unchanged).  The
// code and packing (lower column in the low byte or nibble) were checked
// against the fp64 quantiser on the device.  2^-127 (all-zero blocks, or
// outputs below 2^-118) takes the arithmetic path.
__device__ __forceinline__ void mx_store4(const float *v, int x, int fmt, uint8_t *codes_row, int col) {
    if (x > -127) {
        const float s = __uint_as_float((unsigned)(x + 127) << 23);  // 2^x
        if (fmt == kOutMxFp8E4M3) {
            const float lim = 448.f * s;
            float c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_fmed3f(v[j], -lim, lim);
            mx_short2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(mx_short2{0, 0}, c[0], c[1], s, false);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c[2], c[3], s, true);
            *reinterpret_cast<unsigned *>(codes_row + col) = __builtin_bit_cast(unsigned, w);
        } else {
            unsigned w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], s, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], s, 1);
            *reinterpret_cast<uint16_t *>(codes_row + col / 2) = (uint16_t)w;
        }
        return;
    }
    if (fmt == kOutMxFp8E4M3) {
        const unsigned w = mx_e4m3(ldexpf(v[0], -x)) | (mx_e4m3(ldexpf(v[1], -x)) << 8) |
                           (mx_e4m3(ldexpf(v[2], -x)) << 16) | (mx_e4m3(ldexpf(v[3], -x)) << 24);
        *reinterpret_cast<unsigned *>(codes_row + col) = w;
    } else {
        const unsigned w = mx_e2m1(ldexpf(v[0], -x)) | (mx_e2m1(ldexpf(v[1], -x)) << 4) |
                           (mx_e2m1(ldexpf(v[2], -x)) << 8) | (mx_e2m1(ldexpf(v[3], -x)) << 12);
        *reinterpret_cast<uint16_t *>(codes_row + col / 2) = (uint16_t)w;
    }
}

__device__ __forceinline__ int mx_emax(int fmt) { return fmt == kOutMxFp8E4M3 ? 8 : 2; }

// One 32-column block of a row spread over the 4 lanes lr + 16*lg of a wave,
// as the attention kernels hold it: lane lg has columns 4lg..4lg+3 of each
// 16-column half (v[0..3], v[4..7]).  col = the block's first column.
__device__ __forceinline__ void mx_store_block_4lanes(const float (&v)[8], int fmt, uint8_t *codes_row,
                                                      uint8_t *scales_row, int col, int lg) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = row4_max(amax);
    const int x = mx_block_exp(amax, mx_emax(fmt));
    mx_store4(v, x, fmt, codes_row, col + 4 * lg);
    mx_store4(v + 4, x, fmt, codes_row, col + 16 + 4 * lg);
    if (lg == 0) scales_row[col / 32] = (uint8_t)(x + 127);
}

// One 32-column block over 8 adjacent lanes (lane % 8 = q holds columns
// 4q..4q+3), as the merge kernel holds it.
__device__ __forceinline__ void mx_store_block_8lanes(const float (&v)[4], int fmt, uint8_t *codes_row,
                                                      uint8_t *scales_row, int col, int q) {
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = fmaxf(amax, xor_shuffle(amax, 1));
    amax = fmaxf(amax, xor_shuffle(amax, 2));
    amax = fmaxf(amax, xor_shuffle(amax, 4));
    const int x = mx_block_exp(amax, mx_emax(fmt));
    mx_store4(v, x, fmt, codes_row, col + 4 * q);
    if (q == 0) scales_row[col / 32] = (uint8_t)(x + 127);
}

// One 32-column block over 2 lanes (lane and lane ^ 16, half = 0 / 1 holding
// columns 0..15 / 16..31 of the block, v[4t + j] = column 4t + j of its half),
// as the column-split kernel holds it.
__device__ __forceinline__ void mx_store_block_2lanes(const float (&v)[16], int fmt, uint8_t *codes_row,
                                                      uint8_t *scales_row, int col, int half) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, xor_shuffle(amax, 16));
    const int x = mx_block_exp(amax, mx_emax(fmt));
#pragma unroll
    for (int t = 0; t < 4; ++t) mx_store4(v + 4 * t, x, fmt, codes_row, col + 16 * half + 4 * t);
    if (half == 0) scales_row[col / 32] = (uint8_t)(x + 127);
}

}  // namespace fmha
