// Device-side building blocks shared by the matvec and expert-gather kernels:
// the per-format decode of one 16-byte chunk of packed codes against an x
// slice held in registers, and wavefront reductions.
//
// Formats [S1 = "Stream D - Quantization (FP4 + QAT-int4)...", section 1;
// S2 = "Dense-path int4km coverage + flagship Qwen3.6-35B...", sections 1, 8]:
//   INT4: 32 codes u (nibbles) per 16-byte chunk = one block; w = s * (u - 8)
//   FP4 : 32 E2M1 codes per chunk = one block; w = grid[c] * 2^(e8m0 - 127)
//   INT8: 16 int8 codes per chunk = half a block; w = s * q
//   KM4 : 32 indices per chunk; w = lut[row][c]
// Every decoded value below is exact in fp16 before scaling (the scale is
// applied to the fp32 block sum), so the only rounding is fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

enum Fmt { INT4 = 0, FP4 = 1, INT8 = 2, KM4 = 3 };

constexpr int kWave = 64;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Bytes of codes per chunk is always 16; elements per chunk:
template <int FMT> struct ChunkTraits {
    static constexpr int kElems = (FMT == INT8) ? 16 : 32;
    static constexpr int kXWords = kElems / 2;   // half2 words of x per chunk
};

// x slice for one chunk and one batch row, packed as half2 words in the
// order the decoder consumes them.
//  INT4: word 4d+0 = (x[8d], x[8d+4]), 4d+1 = (x[8d+2], x[8d+6]),
//        4d+2 = (x[8d+1], x[8d+5]), 4d+3 = (x[8d+3], x[8d+7])
//  others: natural pairs (x[2i], x[2i+1]).
template <int FMT>
__device__ __forceinline__ void load_x_slice(const _Float16 *__restrict__ xrow, int chunk, bool valid,
                                             uint32_t (&xw)[ChunkTraits<FMT>::kXWords]) {
    constexpr int E = ChunkTraits<FMT>::kElems;
    if (!valid) {
#pragma unroll
        for (int i = 0; i < E / 2; i++) xw[i] = 0;
        return;
    }
    const uint4 *p = reinterpret_cast<const uint4 *>(xrow + (size_t)chunk * E);
    uint32_t nat[E / 2];
#pragma unroll
    for (int i = 0; i < E / 8; i++) {
        uint4 v = p[i];
        nat[4 * i + 0] = v.x;
        nat[4 * i + 1] = v.y;
        nat[4 * i + 2] = v.z;
        nat[4 * i + 3] = v.w;
    }
    if constexpr (FMT == INT4) {
        // nat[4d + m] = (x[8d+2m], x[8d+2m+1])
#pragma unroll
        for (int d = 0; d < 4; d++) {
            uint32_t a = nat[4 * d + 0], b = nat[4 * d + 1], c = nat[4 * d + 2], e = nat[4 * d + 3];
            // low halves: x0 (a.lo) x2 (b.lo) x4 (c.lo) x6 (e.lo); high: x1 x3 x5 x7
            xw[4 * d + 0] = __builtin_amdgcn_perm(c, a, 0x05040100);  // (x0, x4)
            xw[4 * d + 1] = __builtin_amdgcn_perm(e, b, 0x05040100);  // (x2, x6)
            xw[4 * d + 2] = __builtin_amdgcn_perm(c, a, 0x07060302);  // (x1, x5)
            xw[4 * d + 3] = __builtin_amdgcn_perm(e, b, 0x07060302);  // (x3, x7)
        }
    } else {
#pragma unroll
        for (int i = 0; i < E / 2; i++) xw[i] = nat[i];
    }
}

// ---- per-format chunk dot products: return sum over the chunk of
// ---- (unscaled decoded code) * x in fp32.

// INT4: (w & 0x000F000F) | 0x64006400 is the half2 (1024 + u_lo, 1024 + u_hi);
// the 0x00F0 nibbles land 4 bits higher, i.e. 1024 + 16u. Removing the bias
// exactly gives (u - 8) and 16 (u - 8); the factor 16 is taken out at the end.
__device__ __forceinline__ float chunk_dot_int4(uint4 cw, const uint32_t (&xw)[16]) {
    const h2 b0 = as_h2(0x64086408u);   // (1032, 1032)
    const h2 b1 = as_h2(0x64806480u);   // (1152, 1152)
    float lo = 0.f, hi = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t v = w[d], v8 = v >> 8;
        h2 a04 = as_h2((v & 0x000F000Fu) | 0x64006400u) - b0;
        h2 a15 = as_h2((v & 0x00F000F0u) | 0x64006400u) - b1;
        h2 a26 = as_h2((v8 & 0x000F000Fu) | 0x64006400u) - b0;
        h2 a37 = as_h2((v8 & 0x00F000F0u) | 0x64006400u) - b1;
        lo = dot2(a04, as_h2(xw[4 * d + 0]), lo);
        lo = dot2(a26, as_h2(xw[4 * d + 1]), lo);
        hi = dot2(a15, as_h2(xw[4 * d + 2]), hi);
        hi = dot2(a37, as_h2(xw[4 * d + 3]), hi);
    }
    return __builtin_fmaf(hi, 0.0625f, lo);
}

// FP4: the gfx950 scaled conversion turns one byte (two E2M1 codes, low
// nibble first) into a half2 of grid values; scale 1 keeps them exact.
__device__ __forceinline__ float chunk_dot_fp4(uint4 cw, const uint32_t (&xw)[16]) {
    float acc = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        acc = dot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 0), as_h2(xw[4 * d + 0]), acc);
        acc = dot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 1), as_h2(xw[4 * d + 1]), acc);
        acc = dot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 2), as_h2(xw[4 * d + 2]), acc);
        acc = dot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 3), as_h2(xw[4 * d + 3]), acc);
    }
    return acc;
}

// INT8: bias each byte to u = q + 128, drop it into the mantissa of 1024
// with a byte permute, and subtract 1152: exact q in fp16.
__device__ __forceinline__ float chunk_dot_int8(uint4 cw, const uint32_t (&xw)[8]) {
    const h2 bias = as_h2(0x64806480u);   // (1152, 1152)
    float acc = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t u = w[d] ^ 0x80808080u;
        h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;   // (q0, q1)
        h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;   // (q2, q3)
        acc = dot2(a, as_h2(xw[2 * d + 0]), acc);
        acc = dot2(b, as_h2(xw[2 * d + 1]), acc);
    }
    return acc;
}

// KM4: table lookups from the row's 16-entry fp16 table staged in LDS.
__device__ __forceinline__ float chunk_dot_km4(uint4 cw, const _Float16 *__restrict__ lut,
                                               const uint32_t (&xw)[16]) {
    float acc = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            h2 v;
            v.x = lut[(w[d] >> (8 * i)) & 15u];
            v.y = lut[(w[d] >> (8 * i + 4)) & 15u];
            acc = dot2(v, as_h2(xw[4 * d + i]), acc);
        }
    }
    return acc;
}

// fp16 bits -> fp32 (exact)
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// 2^(byte - 127) as fp32 (byte 0 is the subnormal 2^-127); exact.
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
    return __builtin_ldexpf(1.0f, (int)byte - 127);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64);
// every lane of the group receives the group sum.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, width);
    return v;
}

}  // namespace qmv
