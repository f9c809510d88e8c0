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
//   INT4AFF: 32 codes u per chunk = one block; w = s * u + b (scale and bias
//        per block [S1 sec. 1: affine int4 among the MoE gather formats])
//   INT8KM: 16 byte indices per chunk; w = lut[row / 32][c], one 256-entry
//        table per 32 rows [S3 "Palettization"; S5: int8 k-means, group 32]
// Every decoded value below is exact in fp16 before scaling (the scale is
// applied to the fp32 block sum), so the only rounding is fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

enum Fmt { INT4 = 0, FP4 = 1, INT8 = 2, KM4 = 3, INT4AFF = 4, INT8KM = 5 };

constexpr int kWave = 64;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Bytes of codes per chunk is always 16; elements per chunk:
template <int FMT> struct ChunkTraits {
    static constexpr int kElems = (FMT == INT8 || FMT == INT8KM) ? 16 : 32;
    static constexpr int kXWords = kElems / 2;   // half2 words of x per chunk
};

// x slice for one chunk and one batch row, packed as half2 words in the
// order the decoder consumes them.
//  INT4, INT4AFF: word 4d+0 = (x[8d], x[8d+4]), 4d+1 = (x[8d+2], x[8d+6]),
//        4d+2 = (x[8d+1], x[8d+5]), 4d+3 = (x[8d+3], x[8d+7])
//  others: natural pairs (x[2i], x[2i+1]).
template <int FMT>
__device__ __forceinline__ void load_x_slice(const _Float16 *__restrict__ xrow, int chunk, bool valid,
                                             uint32_t (&xw)[ChunkTraits<FMT>::kXWords]) {
    constexpr int E = ChunkTraits<FMT>::kElems;
    // always load (from chunk 0 when invalid) and zero afterwards: a predicated
    // load would become a branch that serializes the loads around it
    const uint4 *p = reinterpret_cast<const uint4 *>(xrow + (size_t)(valid ? chunk : 0) * E);
    uint32_t nat[E / 2];
#pragma unroll
    for (int i = 0; i < E / 8; i++) {
        uint4 v = p[i];
        nat[4 * i + 0] = valid ? v.x : 0u;
        nat[4 * i + 1] = valid ? v.y : 0u;
        nat[4 * i + 2] = valid ? v.z : 0u;
        nat[4 * i + 3] = valid ? v.w : 0u;
    }
    if constexpr (FMT == INT4 || FMT == INT4AFF) {
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
// (v & mask) | magic as one v_and_or_b32 (the compiler would otherwise emit an
// AND and an OR, since a VOP3 instruction cannot take two literal constants)
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(magic));
    return r;
}

// AFF: the codes are used as u (bias 1024 and 16 * 64 + 1024), not u - 8.
template <bool AFF = false>
__device__ __forceinline__ float chunk_dot_int4(uint4 cw, const uint32_t (&xw)[16]) {
    const h2 b0 = as_h2(AFF ? 0x64006400u : 0x64086408u);   // (1024, 1024) or (1032, 1032)
    const h2 b1 = as_h2(AFF ? 0x64006400u : 0x64806480u);   // (1024, 1024) or (1152, 1152)
    const uint32_t magic = 0x64006400u;
    float lo = 0.f, hi = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t v = w[d], v8 = v >> 8;
        h2 a04 = as_h2(and_or(v, 0x000F000Fu, magic)) - b0;
        h2 a15 = as_h2(and_or(v, 0x00F000F0u, magic)) - b1;
        h2 a26 = as_h2(and_or(v8, 0x000F000Fu, magic)) - b0;
        h2 a37 = as_h2(and_or(v8, 0x00F000F0u, magic)) - b1;
        lo = dot2(a04, as_h2(xw[4 * d + 0]), lo);
        lo = dot2(a26, as_h2(xw[4 * d + 1]), lo);
        hi = dot2(a15, as_h2(xw[4 * d + 2]), hi);
        hi = dot2(a37, as_h2(xw[4 * d + 3]), hi);
    }
    return __builtin_fmaf(hi, 0.0625f, lo);
}

// Sum of the chunk's x values in fp32 (the affine bias multiplies it).
template <int XW>
__device__ __forceinline__ float x_slice_sum(const uint32_t (&xw)[XW]) {
    const h2 one = as_h2(0x3C003C00u);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < XW; i++) s = dot2(as_h2(xw[i]), one, s);
    return s;
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
// Generic form: any table address.
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

// (byte S of w) & 0x1E in one SDWA instruction.
template <int S>
__device__ __forceinline__ uint32_t byte_and_1e(uint32_t w) {
    uint32_t r;
    if constexpr (S == 0)
        asm("v_and_b32_sdwa %0, 30, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(w));
    else if constexpr (S == 1)
        asm("v_and_b32_sdwa %0, 30, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w));
    else if constexpr (S == 2)
        asm("v_and_b32_sdwa %0, 30, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w));
    else
        asm("v_and_b32_sdwa %0, 30, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w));
    return r;
}

// KM4 with the table at a compile-time LDS byte offset: every code's table
// byte offset 2c is one SDWA AND of a pre-shifted code word (w << 1 holds the
// even nibbles at bits 1-4 of each byte, w >> 3 the odd ones), and the row's
// table base folds into the LDS instruction's immediate offset.
// L must be a compile-time constant LDS address after unrolling (a static
// __shared__ array in a one-wave workgroup plus a constant row offset).
__device__ __forceinline__ float chunk_dot_km4_imm(uint4 cw, const char *L, const uint32_t (&xw)[16]) {
    float acc = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t w1 = w[d] << 1, w3 = w[d] >> 3;
        uint32_t a[8] = {byte_and_1e<0>(w1), byte_and_1e<0>(w3), byte_and_1e<1>(w1), byte_and_1e<1>(w3),
                         byte_and_1e<2>(w1), byte_and_1e<2>(w3), byte_and_1e<3>(w1), byte_and_1e<3>(w3)};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            h2 v;
            v.x = *reinterpret_cast<const _Float16 *>(L + a[2 * i]);
            v.y = *reinterpret_cast<const _Float16 *>(L + a[2 * i + 1]);
            acc = dot2(v, as_h2(xw[4 * d + i]), acc);
        }
    }
    return acc;
}

// (byte S of w) << 1: the byte offset of a 2-byte table entry, one SDWA shift.
template <int S>
__device__ __forceinline__ uint32_t byte_shl1(uint32_t w) {
    uint32_t r;
    if constexpr (S == 0)
        asm("v_lshlrev_b32_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(w));
    else if constexpr (S == 1)
        asm("v_lshlrev_b32_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w));
    else if constexpr (S == 2)
        asm("v_lshlrev_b32_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w));
    else
        asm("v_lshlrev_b32_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w));
    return r;
}

// INT8KM: 16 byte indices into a 256-entry fp16 table at the compile-time LDS
// address L (a static __shared__ array of a one-wave workgroup); each byte's
// table offset is one SDWA shift and the table base folds into the LDS
// instruction's immediate offset.
__device__ __forceinline__ float chunk_dot_int8km_imm(uint4 cw, const char *L, const uint32_t (&xw)[8]) {
    float acc = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t a0 = byte_shl1<0>(w[d]), a1 = byte_shl1<1>(w[d]);
        const uint32_t a2 = byte_shl1<2>(w[d]), a3 = byte_shl1<3>(w[d]);
        h2 v, u;
        v.x = *reinterpret_cast<const _Float16 *>(L + a0);
        v.y = *reinterpret_cast<const _Float16 *>(L + a1);
        u.x = *reinterpret_cast<const _Float16 *>(L + a2);
        u.y = *reinterpret_cast<const _Float16 *>(L + a3);
        acc = dot2(v, as_h2(xw[2 * d + 0]), acc);
        acc = dot2(u, as_h2(xw[2 * d + 1]), acc);
    }
    return acc;
}

// INT8KM with a table at any LDS address.
__device__ __forceinline__ float chunk_dot_int8km(uint4 cw, const _Float16 *__restrict__ lut,
                                                  const uint32_t (&xw)[8]) {
    float acc = 0.f;
    uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            h2 v;
            v.x = lut[(w[d] >> (16 * i)) & 255u];
            v.y = lut[(w[d] >> (16 * i + 8)) & 255u];
            acc = dot2(v, as_h2(xw[2 * d + i]), acc);
        }
    }
    return acc;
}

// 16-byte load that bypasses cache allocation (the code planes are streamed once)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Argmax keys: the fp32 value in order-preserving form above the complement
// of the row index, so the largest key is the largest value and, among equal
// values, the lowest row. Every finite value gives a key above 0.
__device__ __forceinline__ uint64_t argmax_key(float v, int64_t row) {
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)row);
}

__device__ __forceinline__ int32_t argmax_key_row(uint64_t k) {
    return (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ float argmax_key_value(uint64_t k) {
    const uint32_t hi = (uint32_t)(k >> 32);
    return __builtin_bit_cast(float, (hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, m), hi = __shfl_xor((uint32_t)(k >> 32), m);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

// Sum over each row of 16 lanes with DPP (quad swaps, half-row mirror, row
// mirror); every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    return v;
}

// Cross-half exchange-and-add without LDS. v_permlane32_swap swaps the upper
// 32 lanes of its first operand with the lower 32 of its second, so adding the
// two results gives a(l) + a(l + 32) in lanes 0..31 and b(l - 32) + b(l) in
// lanes 32..63; v_permlane16_swap does the same between 16-lane rows 0/1 and
// 2/3 (a in rows 0 and 2, b in rows 1 and 3). The empty asm keeps the second
// result opaque: without it the optimizer folds the float reinterpretation of
// the second result into the first and adds the first to itself.
template <int HALF>
__device__ __forceinline__ float half_swap_add(float a, float b) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    u32x2 s;
    if constexpr (HALF == 32) s = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
    else s = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
    uint32_t s0 = s[0], s1 = s[1];
    __asm__("" : "+v"(s1));
    return __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
}

// Reduce V partial sums per lane over groups of LPR lanes (LPR = 16, 32 or 64).
// Instead of V separate butterflies, each cross-row step exchanges half of the
// values and keeps the other half ("transposed" reduction), so a step costs
// V/2 lane swaps and the set of live values halves. On return v[0 .. live) hold
// group sums, identical in every lane of a 16-lane row; value j of lane l is
// the original index base + j (see live/base below).
template <int V, int LPR>
struct GroupReduce {
    static constexpr bool kH32 = (LPR == 64 && V >= 2);
    static constexpr int kV1 = kH32 ? V / 2 : V;
    static constexpr bool kH16 = (LPR >= 32 && kV1 >= 2);
    static constexpr int live = kH16 ? kV1 / 2 : kV1;

    __device__ __forceinline__ static void run(float (&v)[V], int /*lane*/) {
        if constexpr (kH32) {
#pragma unroll
            for (int j = 0; j < V / 2; j++) v[j] = half_swap_add<32>(v[j], v[j + V / 2]);
        } else if constexpr (LPR == 64) {
            v[0] = half_swap_add<32>(v[0], v[0]);
        }
        if constexpr (kH16) {
#pragma unroll
            for (int j = 0; j < kV1 / 2; j++) v[j] = half_swap_add<16>(v[j], v[j + kV1 / 2]);
        } else if constexpr (LPR >= 32) {
            v[0] = half_swap_add<16>(v[0], v[0]);
        }
#pragma unroll
        for (int j = 0; j < live; j++) v[j] = row16_sum(v[j]);
    }
    // original index of v[0] in this lane
    __device__ __forceinline__ static int base(int lane) {
        int b = 0;
        if constexpr (kH32) b += (lane & 32) ? V / 2 : 0;
        if constexpr (kH16) b += (lane & 16) ? kV1 / 2 : 0;
        return b;
    }
    // true for the one lane per (16-lane row, distinct value set) that stores
    __device__ __forceinline__ static bool writer(int lane) {
        if (lane & 15) return false;
        if constexpr (LPR == 64 && !kH32) { if (lane & 32) return false; }
        if constexpr (LPR >= 32 && !kH16) { if (lane & 16) return false; }
        return true;
    }
};

}  // namespace qmv
