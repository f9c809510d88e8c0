// Batched decode matvec on the matrix cores: y[b][n] = sum_k dequant(W)[n][k]
// * x[b][k] for a batch of up to 8 tokens ("Dense-path int4km coverage +
// flagship Qwen3.6-35B - session findings & methods", sections 1 and 8: the
// fused dequant-matvec at decode batch sizes; the next step the page lists
// is the batched B = 4-8 form).
//
// gfx950 design. At batch b the dot2 path spends b times the VALU work of
// batch 1 on multiplies while the decode work stays the same; here the
// multiplies go to v_mfma_f32_16x16x32_f16, which takes 16 weight rows x 32
// k against 16 batch columns per instruction, so the VALU only decodes.
//   - Operands: A = x (16 batch rows, rows >= B read zeros), B = the
//     decoded weights (32 k x 16 rows). Result D[batch][row]: lane (r, q),
//     r = lane % 16, q = lane / 16, holds rows r, batches 4q .. 4q + 3.
//   - Every lane of row r owns row r, so one MFMA result per block is scaled
//     by that lane's own block scale (fp32 FMA) before accumulation; the
//     decoded values stay exact in fp16 as in the dot2 path. The 16 rows of
//     one MFMA all take the same 32-k block. km4 has no block scale: its
//     MFMAs accumulate directly, and each lane holds its row's table in
//     registers as byte planes, looked up with v_perm (no LDS reads).
//   - Codes reach the MFMA layout through a small per-wave LDS stage (global
//     loads stay whole cache lines): lane (r, q) takes 16-byte chunk 4j + q
//     of row r, and a 4 x 4 dword transpose across the four 16-lane rows
//     (permlane32/16 swaps) gives it dword q of chunks 4j .. 4j + 3, exactly
//     its share of the four MFMAs of those blocks (int8: two blocks of two
//     chunks each).
//   - x is staged once per workgroup in LDS, in the element order the
//     decoder produces, one row per batch token, each row padded by 16 bytes
//     so the 16 batch lanes of a read hit distinct banks.
#include "qmv_device.h"
#include "qmv_launch.h"

namespace qmv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

constexpr int kMfmaWaves = 4;

// Lane (r, q) holds X[q][m] in w[m] (chunk q, dword m); afterwards it holds
// X[m][q] (dword q of chunk m). permlane32_swap exchanges the upper two
// 16-lane rows of its first operand with the lower two of its second;
// permlane16_swap the odd rows of its first operand with the even rows of
// its second.
__device__ __forceinline__ void transpose4(uint32_t (&w)[4]) {
    u2v s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    u2v s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    u2v s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    u2v s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    w[0] = s01[0];
    w[1] = s01[1];
    w[2] = s23[0];
    w[3] = s23[1];
}

__device__ __forceinline__ h8 h8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    u4v v = {a, b, c, d};
    return __builtin_bit_cast(h8, v);
}

// 8 weights of one 32-k block for one lane, in the order x is staged:
//  INT4: one dword (nibbles n0..n7) -> n0 n4 n1 n5 n2 n6 n3 n7
//  FP4 : one dword -> c0 .. c7
//  INT8: two dwords (codes 4q..4q+3 and 16+4q..16+4q+3 of the block)
template <int FMT>
__device__ __forceinline__ h8 decode8(uint32_t v, uint32_t v2) {
    if constexpr (FMT == INT4 || FMT == INT4AFF) {
        // int4: u - 8; affine int4: u (its bias is added per block)
        const h2 b0 = as_h2(FMT == INT4 ? 0x64086408u : 0x64006400u);   // (1032, 1032) or (1024, 1024)
        const uint32_t magic = 0x64006400u;
        h2 a0 = as_h2(and_or(v, 0x000F000Fu, magic)) - b0;
        h2 a1 = as_h2(and_or(v >> 4, 0x000F000Fu, magic)) - b0;
        h2 a2 = as_h2(and_or(v >> 8, 0x000F000Fu, magic)) - b0;
        h2 a3 = as_h2(and_or(v >> 12, 0x000F000Fu, magic)) - b0;
        return h8_of(as_u32(a0), as_u32(a1), as_u32(a2), as_u32(a3));
    } else if constexpr (FMT == FP4) {
        return h8_of(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0)),
                     as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1)),
                     as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2)),
                     as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3)));
    } else {
        const h2 bias = as_h2(0x64806480u);   // (1152, 1152)
        uint32_t u = v ^ 0x80808080u, u2 = v2 ^ 0x80808080u;
        h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;
        h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;
        h2 c = as_h2(__builtin_amdgcn_perm(0x64646464u, u2, 0x04010400u)) - bias;
        h2 d = as_h2(__builtin_amdgcn_perm(0x64646464u, u2, 0x04030402u)) - bias;
        return h8_of(as_u32(a), as_u32(b), as_u32(c), as_u32(d));
    }
}

// KM4 from registers: the lane's row table as byte planes, L[k] = low bytes
// and H[k] = high bytes of entries 4k .. 4k + 3. One v_perm looks up four
// codes in an 8-entry byte plane (selector = code & 7); entries 8..15 come
// from the second pair of planes and a byte-wise select on bit 3 of the code
// (v_perm's sign-replicating selectors spread that bit over its byte).
// Result order c0 c2 c1 c3 c4 c6 c5 c7 (x is staged to match). No LDS access:
// sixteen rows' tables looked up from LDS in one instruction meet bank
// conflicts, which limited the LDS form to about half this rate.
__device__ __forceinline__ uint32_t bsel(uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); }
__device__ __forceinline__ h8 decode8_km4_reg(uint32_t w, const uint32_t (&L)[4], const uint32_t (&H)[4]) {
    const uint32_t se = w & 0x07070707u;            // even codes c0 c2 c4 c6, low 3 bits
    const uint32_t so = (w >> 4) & 0x07070707u;     // odd codes c1 c3 c5 c7
    // 0xFF where bit 3 of the code is set: selectors 8..11 replicate bit 15 /
    // 31 of the second / first operand
    const uint32_t me = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);   // bits 3, 11, 19, 27
    const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);         // bits 7, 15, 23, 31
    const uint32_t le = bsel(me, __builtin_amdgcn_perm(L[3], L[2], se), __builtin_amdgcn_perm(L[1], L[0], se));
    const uint32_t he = bsel(me, __builtin_amdgcn_perm(H[3], H[2], se), __builtin_amdgcn_perm(H[1], H[0], se));
    const uint32_t lo = bsel(mo, __builtin_amdgcn_perm(L[3], L[2], so), __builtin_amdgcn_perm(L[1], L[0], so));
    const uint32_t ho = bsel(mo, __builtin_amdgcn_perm(H[3], H[2], so), __builtin_amdgcn_perm(H[1], H[0], so));
    return h8_of(__builtin_amdgcn_perm(he, le, 0x05010400u), __builtin_amdgcn_perm(ho, lo, 0x05010400u),
                 __builtin_amdgcn_perm(he, le, 0x07030602u), __builtin_amdgcn_perm(ho, lo, 0x07030602u));
}

// INT8KM: the 8 byte codes of two dwords (the INT8 element order) looked up
// in the row group's 256-entry table in LDS at byte address tbase: one SDWA
// shift and one add per code form the address.
__device__ __forceinline__ _Float16 lds_half(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) _Float16 *>((size_t)addr);
}
__device__ __forceinline__ h8 decode8_km8(uint32_t w0, uint32_t w1, uint32_t tbase) {
    h2 v0, v1, v2, v3;
    v0.x = lds_half(tbase + byte_shl1<0>(w0));
    v0.y = lds_half(tbase + byte_shl1<1>(w0));
    v1.x = lds_half(tbase + byte_shl1<2>(w0));
    v1.y = lds_half(tbase + byte_shl1<3>(w0));
    v2.x = lds_half(tbase + byte_shl1<0>(w1));
    v2.y = lds_half(tbase + byte_shl1<1>(w1));
    v3.x = lds_half(tbase + byte_shl1<2>(w1));
    v3.y = lds_half(tbase + byte_shl1<3>(w1));
    return h8_of(as_u32(v0), as_u32(v1), as_u32(v2), as_u32(v3));
}

// One 8-element x group (16 bytes) in decoder order; group g of a row is
// staged at halfs 8g .. 8g + 7. For INT8, group 4c + q holds elements
// 32c + 4q .. +3 and 32c + 16 + 4q .. +3.
template <int FMT>
__device__ __forceinline__ uint4 stage_group(const _Float16 *__restrict__ xrow, int g) {
    if constexpr (FMT == INT8 || FMT == INT8KM) {
        const int c = g >> 2, q = g & 3;
        uint2 lo = *reinterpret_cast<const uint2 *>(xrow + 32 * c + 4 * q);
        uint2 hi = *reinterpret_cast<const uint2 *>(xrow + 32 * c + 16 + 4 * q);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        uint4 v = *reinterpret_cast<const uint4 *>(xrow + 8 * g);
        if constexpr (FMT == KM4) {
            // (x0 x1)(x2 x3)(x4 x5)(x6 x7) -> (x0 x2)(x1 x3)(x4 x6)(x5 x7)
            return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                              __builtin_amdgcn_perm(v.w, v.z, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
        }
        if constexpr (FMT == INT4 || FMT == INT4AFF) {
            // (x0 x1)(x2 x3)(x4 x5)(x6 x7) -> (x0 x4)(x1 x5)(x2 x6)(x3 x7)
            return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                              __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
        }
        return v;
    }
}

// Per-wave LDS staging of one row group (16 rows): the codes of one load
// step (16 rows x 256 bytes, rows padded by 16 bytes) and the group's scale
// rows (padded by 8 or 4 bytes), so that the MFMA-layout reads hit distinct
// banks; plus 256 zero bytes per workgroup for the A operand of batch lanes
// >= B.
constexpr int kCodeRowLds = 256 + 16;
constexpr bool kLdsCodes = true;   // staged loads measured faster on MI355X
constexpr int kZeroLds = 256;
template <int FMT> constexpr int scale_pad() {
    return (FMT == INT4) ? 8 : (FMT == INT4AFF ? 16 : ((FMT == KM4 || FMT == INT8KM) ? 0 : 4));
}
// per-row bytes of the scale plane (KM4: the row's 16-entry fp16 table;
// INT4AFF: a 32-bit scale + bias word per block)
template <int FMT> __host__ __device__ constexpr int scale_row_bytes(int K) {
    // INT8KM: a row group's 256-entry table, 512 bytes over 16 rows
    return (FMT == KM4 || FMT == INT8KM) ? 32 : ((FMT == FP4) ? K / 32 : (FMT == INT4AFF ? K / 8 : K / 16));
}
// affine int4: per-workgroup LDS table of the x block sums, [K/32][16 batch] fp32
template <int FMT> __host__ __device__ constexpr int xsum_lds_bytes(int K) {
    return (FMT == INT4AFF) ? (K / 32) * 16 * 4 : 0;
}
template <int FMT, bool LDS_CODES> __host__ __device__ constexpr int wave_lds_bytes(int K) {
    return (LDS_CODES ? 16 * kCodeRowLds : 0) + ((16 * (scale_row_bytes<FMT>(K) + scale_pad<FMT>()) + 15) / 16) * 16;
}
// 16-byte pieces per lane of a group's scales (16 rows x scale_row_bytes)
template <int FMT> __host__ __device__ constexpr int scale_pieces(int K) {
    return (16 * scale_row_bytes<FMT>(K) + 1023) / 1024;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Each wave streams RG row groups of 16 rows. A load step covers 256 bytes
// of every row of the group (four j-steps), read as four instructions of four
// rows x 256 contiguous bytes (whole cache lines), and goes through LDS into
// the MFMA layout (lane (r, q): chunk 4j + q of row r). A group's scales are
// one contiguous stretch of the scale plane (SP 16-byte pieces per lane),
// read whole with the group's first step. Loads run D steps ahead of the
// arithmetic in a ring of registers, which keeps enough bytes in flight per
// wave to cover the memory latency.
template <int FMT, int RG, int SP, int D, bool LDS_CODES>
__global__ __launch_bounds__(64 * kMfmaWaves) void mv_mfma(const uint8_t *__restrict__ codes,
                                                          const void *__restrict__ plane, int64_t N, int K,
                                                          const _Float16 *__restrict__ x, int B,
                                                          float *__restrict__ y, uint64_t *__restrict__ hdr) {
    extern __shared__ __align__(16) _Float16 xs[];
    // fused argmax: the first workgroup zeroes the reduction header
    if (hdr != nullptr && blockIdx.x == 0 && threadIdx.x < kArgmaxHeader) hdr[threadIdx.x] = 0;
    constexpr bool BYTES = (FMT == INT8 || FMT == INT8KM);   // one code per byte
    constexpr bool TABLE = (FMT == KM4 || FMT == INT8KM);   // no block scales
    constexpr int MPJ = BYTES ? 2 : 4;                      // blocks (MFMAs) per j-step
    const int KP = K + 8;                         // padded x row in LDS, halfs
    const int groups = K / 8;
    for (int i = threadIdx.x; i < B * groups; i += 64 * kMfmaWaves) {
        const int b = i / groups, g = i - b * groups;
        *reinterpret_cast<uint4 *>(xs + b * KP + 8 * g) = stage_group<FMT>(x + (size_t)b * K, g);
    }
    uint8_t *const zl = reinterpret_cast<uint8_t *>(xs + B * KP);
    if (threadIdx.x < kZeroLds / 16) reinterpret_cast<uint4 *>(zl)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    float *const xsum_l = reinterpret_cast<float *>(zl + kZeroLds);
    if constexpr (FMT == INT4AFF) {
        // the affine bias multiplies the block sum of x: [block][batch], batches >= B zero
        for (int i = threadIdx.x; i < (K / 32) * 16; i += 64 * kMfmaWaves) {
            const int blk = i >> 4, b = i & 15;
            float sum = 0.f;
            if (b < B) {
                const uint4 *p = reinterpret_cast<const uint4 *>(x + (size_t)b * K + 32 * blk);
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const uint4 v = p[u];
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; e++) sum = dot2(as_h2(w4[e]), as_h2(0x3C003C00u), sum);
                }
            }
            xsum_l[i] = sum;
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar branches
    const int r = lane & 15, q = lane >> 4;
    const int64_t rows0 = ((int64_t)blockIdx.x * kMfmaWaves + wave) * (RG * 16);
    if (rows0 >= N) return;
    const int J = BYTES ? K / 64 : K / 128;   // j-steps per row
    const int cpr = 4 * J;                             // 16-byte chunks per row
    const uint32_t row_bytes = BYTES ? (uint32_t)K : (uint32_t)K / 2;
    const int srb = scale_row_bytes<FMT>(K);
    const int srs = srb + scale_pad<FMT>();            // padded scale row in LDS
    uint8_t *wl = zl + kZeroLds + xsum_lds_bytes<FMT>(K) + wave * wave_lds_bytes<FMT, LDS_CODES>(K);
    uint8_t *cl = wl;                                       // codes [16][kCodeRowLds]
    uint8_t *sl = wl + (LDS_CODES ? 16 * kCodeRowLds : 0);  // scales [16][srs]
    // A operand of j-step j: xa + xstride * j, then 64 bytes per block. Batch
    // lanes >= B read the zero bytes with stride 0.
    const uint8_t *xa = (r < B) ? reinterpret_cast<const uint8_t *>(xs + r * KP + 8 * q) : zl + 16 * q;
    const uint32_t xstride = (r < B) ? 64u * MPJ : 0u;
    const int steps_per_group = (J + 3) / 4;
    const int nsteps = RG * steps_per_group;

    // Every step issues the same loads unconditionally (a branch around a
    // load makes the compiler wait for all outstanding loads where the paths
    // join, which would drain the ring): steps past the end reload the last
    // step, and steps that do not start a group read their scale pieces from
    // one uniform address (a single cached request).
    uint4 cw[D][4];
    uint4 sc[D][SP];
    auto issue = [&](int s_in, uint4 (&c)[4], uint4 (&sv)[SP]) {
        const int s = s_in < nsteps ? s_in : nsteps - 1;
        const int g = s / steps_per_group;
        const int t = s - g * steps_per_group;
        const int64_t grow = rows0 + g * 16;
        // wave-uniform base, 32-bit lane offsets; rows past N read row N - 1
        const int64_t growc = grow < N ? grow : N - 1;
        const int lim = (int)(N - 1 - growc < 15 ? N - 1 - growc : 15);
        const uint8_t *cbase = codes + growc * (int64_t)row_bytes;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            // staged: four rows x 256 bytes per instruction; direct: lane (r, q)
            // takes chunk 4j + q of row r of j-step j = 4t + i
            int rr = LDS_CODES ? 4 * i + (lane >> 4) : r;
            rr = rr < lim ? rr : lim;
            int ch = LDS_CODES ? 16 * t + (lane & 15) : 16 * t + 4 * i + q;
            ch = ch < cpr ? ch : 0;   // past the row end: any valid chunk, never used
            c[i] = load_stream16(cbase + ((uint32_t)rr * row_bytes + (uint32_t)ch * 16u));
        }
        // the scale rows of 16 consecutive rows are contiguous: 16 * srb
        // bytes. A last, partial group reads rows N - 16 .. N - 1 instead
        // (N >= 16) and looks its rows up shifted by the difference.
        const int64_t g0 = grow + 16 <= N ? grow : N - 16;
        // int8km: the table of the row group's 32-row group (N % 32 == 0, so no partial groups)
        const uint8_t *sp = reinterpret_cast<const uint8_t *>(plane) + (FMT == INT8KM ? (g0 / 32) * 512 : g0 * srb);
#pragma unroll
        for (int u = 0; u < SP; u++) {
            int off = 16 * (lane + 64 * u);
            off = (t == 0 && off + 16 <= 16 * srb) ? off : 0;
            sv[u] = *reinterpret_cast<const uint4 *>((t == 0) ? sp + off : reinterpret_cast<const uint8_t *>(plane));
        }
    };

#pragma unroll
    for (int u = 0; u < D; u++) issue(u, cw[u], sc[u]);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    f4 kacc[MPJ];
#pragma unroll
    for (int m = 0; m < MPJ; m++) kacc[m] = f4{0.f, 0.f, 0.f, 0.f};
    uint32_t kL[4] = {0u, 0u, 0u, 0u}, kH[4] = {0u, 0u, 0u, 0u};   // km4: the lane's row table as byte planes
    for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
        for (int u = 0; u < D; u++) {
            // The loads are issued on every path (no early exit between them):
            // where paths with different loads in flight join, the compiler
            // must wait for all of them, which would drain the ring. Steps past
            // the end only skip their LDS work and arithmetic.
            const int s = s0 + u;
            const int sc_step = s < nsteps ? s : nsteps - 1;
            const int g = sc_step / steps_per_group;
            const int t = sc_step - g * steps_per_group;
            const int64_t grow = rows0 + g * 16;
            const bool valid = s < nsteps && grow < N;
            if (valid) {
                // stage this step's codes (and at a group's first step its scales)
                if constexpr (LDS_CODES) {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        *reinterpret_cast<uint4 *>(cl + (4 * i + (lane >> 4)) * kCodeRowLds + (lane & 15) * 16) =
                            cw[u][i];
                }
                if (t == 0) {
#pragma unroll
                    for (int v = 0; v < SP; v++) {
                        const uint32_t wv[4] = {sc[u][v].x, sc[u][v].y, sc[u][v].z, sc[u][v].w};
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int off = 16 * (lane + 64 * v) + 4 * e;   // byte offset in the group's scales
                            if (off < 16 * srb) {
                                const int row = off / srb, col = off - row * srb;
                                *reinterpret_cast<uint32_t *>(sl + row * srs + col) = wv[e];
                            }
                        }
                    }
                }
            }
            wave_sync_lds();
            uint4 cu[4];
#pragma unroll
            for (int i = 0; i < 4; i++) cu[i] = cw[u][i];
            issue(s + D, cw[u], sc[u]);
            if (valid) {
                // LDS scale row of this lane's row (see the partial-group note above)
                const int delta = (int)(grow + 16 <= N ? 0 : grow - (N - 16));
                const int srow = r + delta < 16 ? r + delta : 15;
                if constexpr (FMT == KM4) {
                    if (t == 0) {
                        // entries 2i, 2i + 1 in dword i; split into low / high byte planes
                        const uint4 a = *reinterpret_cast<const uint4 *>(sl + srow * srs);
                        const uint4 b = *reinterpret_cast<const uint4 *>(sl + srow * srs + 16);
                        const uint32_t tw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                        for (int k = 0; k < 4; k++) {
                            kL[k] = __builtin_amdgcn_perm(tw[2 * k + 1], tw[2 * k], 0x06040200u);
                            kH[k] = __builtin_amdgcn_perm(tw[2 * k + 1], tw[2 * k], 0x07050301u);
                        }
                    }
                }
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const int j = 4 * t + jj;   // J % 4 == 0: no partial steps
                    const uint4 c4 =
                        LDS_CODES ? *reinterpret_cast<const uint4 *>(cl + r * kCodeRowLds + (4 * jj + q) * 16) : cu[jj];
                    uint32_t w[4] = {c4.x, c4.y, c4.z, c4.w};
                    transpose4(w);
                    uint32_t s0w = 0, s1w = 0;
                    uint4 s4 = make_uint4(0u, 0u, 0u, 0u);
                    if constexpr (FMT == INT4AFF) {
                        s4 = *reinterpret_cast<const uint4 *>(sl + srow * srs + 16 * j);
                    } else if constexpr (FMT == INT4) {
                        const uint2 s2 = *reinterpret_cast<const uint2 *>(sl + srow * srs + 8 * j);
                        s0w = s2.x;
                        s1w = s2.y;
                    } else if constexpr (!TABLE) {
                        s0w = *reinterpret_cast<const uint32_t *>(sl + srow * srs + 4 * j);
                    }
                    // the j-step's MFMAs are independent: decode and read every
                    // operand first, issue the MFMAs back to back, then scale
                    // and accumulate
                    h8 ax[MPJ], bw[MPJ];
                    f4 d[MPJ];
#pragma unroll
                    for (int m = 0; m < MPJ; m++) {
                        ax[m] = *reinterpret_cast<const h8 *>(xa + xstride * (uint32_t)j + 64 * m);
                        if constexpr (FMT == KM4)
                            bw[m] = decode8_km4_reg(w[m], kL, kH);
                        else if constexpr (FMT == INT8KM)
                            bw[m] = decode8_km8(w[2 * m], w[2 * m + 1], (uint32_t)(uintptr_t)sl);
                        else
                            bw[m] = (FMT == INT8) ? decode8<FMT>(w[2 * m], w[2 * m + 1]) : decode8<FMT>(w[m], 0u);
                    }
                    if constexpr (TABLE) {
                        // no block scales: the MFMAs accumulate directly (one
                        // accumulator per block position keeps them independent)
#pragma unroll
                        for (int m = 0; m < MPJ; m++)
                            kacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax[m], bw[m], kacc[m], 0, 0, 0);
                        continue;
                    }
#pragma unroll
                    for (int m = 0; m < MPJ; m++) {
                        const f4 zero = {0.f, 0.f, 0.f, 0.f};
                        d[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax[m], bw[m], zero, 0, 0, 0);
                    }
#pragma unroll
                    for (int m = 0; m < MPJ; m++) {
                        float scl;
                        if constexpr (FMT == INT4AFF) {
                            const uint32_t sb = (m == 0) ? s4.x : (m == 1) ? s4.y : (m == 2) ? s4.z : s4.w;
                            scl = f16_bits_to_f32((uint16_t)(sb & 0xFFFFu));
                            const float bia = f16_bits_to_f32((uint16_t)(sb >> 16));
                            const f4 xsm = *reinterpret_cast<const f4 *>(xsum_l + (4 * j + m) * 16 + 4 * q);
#pragma unroll
                            for (int v = 0; v < 4; v++) acc[v] = __builtin_fmaf(xsm[v], bia, acc[v]);
                        } else if constexpr (FMT == INT4) {
                            const uint32_t pr = (m < 2) ? s0w : s1w;
                            scl = f16_bits_to_f32((uint16_t)((m & 1) ? (pr >> 16) : (pr & 0xFFFFu)));
                        } else if constexpr (FMT == FP4) {
                            scl = e8m0_to_f32((s0w >> (8 * m)) & 0xFFu);
                        } else {
                            scl = f16_bits_to_f32((uint16_t)(m ? (s0w >> 16) : (s0w & 0xFFFFu)));
                        }
#pragma unroll
                        for (int v = 0; v < 4; v++) acc[v] = __builtin_fmaf(d[m][v], scl, acc[v]);
                    }
                }
            }
            wave_sync_lds();   // the next step rewrites the staging buffers
            if (valid && t == steps_per_group - 1) {
                // group done: lane (r, q) holds y[4q + v][row]
                if constexpr (TABLE) {
#pragma unroll
                    for (int m = 0; m < MPJ; m++) {
#pragma unroll
                        for (int v = 0; v < 4; v++) acc[v] += kacc[m][v];
                        kacc[m] = f4{0.f, 0.f, 0.f, 0.f};
                    }
                }
                const int64_t row = grow + r;
                if (row < N) {
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        if (4 * q + v < B) y[(size_t)(4 * q + v) * N + row] = acc[v];
                }
                acc = f4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// km4 at batch 3-4 on 4x4x4 matrix-core blocks (v_mfma_f32_4x4x4_16b_f16:
// 16 independent 4 x 4 x 4 products per instruction). Lane 4b + j belongs to
// block b: it supplies row j of the block's A (tokens x 4 k), column j of its
// B (4 k x weight rows) and receives column j of its D (tokens x weight rows,
// token i in register i). Block b takes the 32-code chunks b, 16 + b, 32 + b,
// ... of every weight row, so one instruction spans only 4 weight rows: their
// 16-entry fp16 tables (4 x 32 bytes) cover the 32 LDS banks once and every
// lane looks its codes up in LDS without bank conflicts, where the 16 rows of
// a 16 x 16 operand meet in the banks (the register-table decode above costs
// 3 VALU per code; this one about 2 plus one LDS read). Per code the VALU
// puts the code's byte offset into the lane's row-table base (one SDWA OR of
// a pre-masked code word) and pairs two fp16 values for the B operand. The
// 16 block sums of a row are added across lanes at the end.
// x is staged once per workgroup in LDS as [token][chunk][36 halfs] with 16
// more halfs after each token row: the 64 lanes of an A-operand read (16
// chunks x 4 tokens, 8 bytes each) then fall on distinct bank pairs, where an
// unpadded token stride (a multiple of 32 dwords) put the four tokens of a
// chunk on the same banks and doubled the LDS time at batch 8.
// Each wave owns Q quads of 4 rows per group and strides over the groups;
// an x read serves the Q quads of its step.
// Measured on MI355X (HIP graphs, 248320 x 2048 cycling 4 weight copies):
// B = 3 / 4 59.2 / 60.3 us against 76.0 / 78.2 us for mv_mfma; at 16384 to
// 124160 rows 8-25% faster. At B = 8 (two token quads, twice the MFMAs and x
// reads) it only matched mv_mfma (72.2-76.8 against 74.9-77.4 us), and at
// B = 2 the dot2 kernel is as fast, so it takes B = 3, 4 only.
// ---------------------------------------------------------------------------
typedef _Float16 h4q __attribute__((ext_vector_type(4)));
constexpr int kQuadWaves = 8;       // waves per workgroup, sharing one x stage
constexpr int kQuadXChunk = 36;     // halfs per staged 32-element x chunk
constexpr int kQuadXRowPad = 16;    // halfs after each staged token row

// base | (byte S of m): the table byte address of one pre-masked code, one SDWA OR
template <int S>
__device__ __forceinline__ uint32_t or_code_byte(uint32_t base, uint32_t m) {
    uint32_t r;
    if constexpr (S == 0)
        asm("v_or_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(base), "v"(m));
    else if constexpr (S == 1)
        asm("v_or_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(base), "v"(m));
    else if constexpr (S == 2)
        asm("v_or_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(base), "v"(m));
    else
        asm("v_or_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(base), "v"(m));
    return r;
}
__device__ __forceinline__ uint32_t lds_u16(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t *>((size_t)addr);
}
__device__ __forceinline__ h4q lds_h4(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) h4q *>((size_t)addr);
}
__host__ __device__ constexpr int quad_x_row(int K) { return (K / 32) * kQuadXChunk + kQuadXRowPad; }

template <int Q, int KC, int BQ = 1>   // K = 512 * KC; BQ token quads
__global__ __launch_bounds__(64 * kQuadWaves) void mv_km4_quad(const uint8_t *__restrict__ codes,
                                                               const uint16_t *__restrict__ lut, int64_t N,
                                                               const _Float16 *__restrict__ x, int B,
                                                               float *__restrict__ y, uint64_t *__restrict__ hdr) {
    constexpr int K = 512 * KC, ROWS = 4 * Q, NT = 4 * BQ, XROW = quad_x_row(K);
    constexpr int TW = (ROWS * 8 + 63) / 64;   // table dwords per lane per group
    extern __shared__ __align__(16) uint8_t qlds[];
    // fused argmax: the first workgroup zeroes the reduction header
    if (hdr != nullptr && blockIdx.x == 0 && threadIdx.x < kArgmaxHeader) hdr[threadIdx.x] = 0;
    _Float16 *xs = reinterpret_cast<_Float16 *>(qlds);
    for (int i = threadIdx.x; i < NT * (K / 4); i += 64 * kQuadWaves) {
        const int b = i / (K / 4), k = 4 * (i - b * (K / 4));
        uint2 v = make_uint2(0u, 0u);   // tokens >= B read zeros
        if (b < B) v = *reinterpret_cast<const uint2 *>(x + (size_t)b * K + k);
        *reinterpret_cast<uint2 *>(xs + b * XROW + (k >> 5) * kQuadXChunk + (k & 31)) = v;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int blk = lane >> 2, j = lane & 3;
    // per-wave tables [ROWS][16] fp16 (32-byte aligned: the code offsets are OR-ed in)
    uint8_t *tab = qlds + NT * XROW * 2 + wave * (ROWS * 32);
    const uint32_t rb = (uint32_t)(uintptr_t)tab + 32u * j;   // row j of quad 0
    const uint32_t xa = (uint32_t)(uintptr_t)xs + (uint32_t)((j * XROW + blk * kQuadXChunk) * 2);
    const int64_t ngroups = (N + ROWS - 1) / ROWS;
    for (int64_t g = (int64_t)blockIdx.x * kQuadWaves + wave; g < ngroups; g += (int64_t)gridDim.x * kQuadWaves) {
        const int64_t row0 = g * ROWS;
        // rows past N read row N - 1 and are never stored
        uint32_t tv[TW];
#pragma unroll
        for (int q = 0; q < TW; q++) {
            const int i = q * 64 + lane;
            const int64_t r = row0 + (i >> 3) < N ? row0 + (i >> 3) : N - 1;
            tv[q] = reinterpret_cast<const uint32_t *>(lut)[r * 8 + (i & 7)];
        }
        uint4 cw[Q][KC];
#pragma unroll
        for (int u = 0; u < Q; u++) {
            const int64_t r = row0 + 4 * u + j < N ? row0 + 4 * u + j : N - 1;
#pragma unroll
            for (int kc = 0; kc < KC; kc++)
                cw[u][kc] = load_stream16(codes + r * (K / 2) + (uint32_t)(16 * kc + blk) * 16u);
        }
#pragma unroll
        for (int q = 0; q < TW; q++) {
            const int i = q * 64 + lane;
            if (i < ROWS * 8) reinterpret_cast<uint32_t *>(tab)[i] = tv[q];
        }
        wave_sync_lds();
        f4 acc[Q][BQ];
#pragma unroll
        for (int u = 0; u < Q; u++)
#pragma unroll
            for (int p = 0; p < BQ; p++) acc[u][p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
#pragma unroll
            for (int d = 0; d < 4; d++) {
                // codes 8d .. 8d + 7 of the chunk: two k-steps of 4
                h4q x0[BQ], x1[BQ];
#pragma unroll
                for (int p = 0; p < BQ; p++) {
                    x0[p] = lds_h4(xa + (uint32_t)((p * 4 * XROW + 16 * kc * kQuadXChunk + 8 * d) * 2));
                    x1[p] = lds_h4(xa + (uint32_t)((p * 4 * XROW + 16 * kc * kQuadXChunk + 8 * d + 4) * 2));
                }
#pragma unroll
                for (int u = 0; u < Q; u++) {
                    const uint32_t w = (d == 0) ? cw[u][kc].x : (d == 1) ? cw[u][kc].y : (d == 2) ? cw[u][kc].z : cw[u][kc].w;
                    // byte offsets 2c of the even (low nibble) and odd codes
                    const uint32_t ml = (w << 1) & 0x1E1E1E1Eu, mh = (w >> 3) & 0x1E1E1E1Eu;
                    const uint32_t ub = rb + 128u * u;
                    const uint32_t t0 = lds_u16(or_code_byte<0>(ub, ml)), t1 = lds_u16(or_code_byte<0>(ub, mh));
                    const uint32_t t2 = lds_u16(or_code_byte<1>(ub, ml)), t3 = lds_u16(or_code_byte<1>(ub, mh));
                    const uint32_t t4 = lds_u16(or_code_byte<2>(ub, ml)), t5 = lds_u16(or_code_byte<2>(ub, mh));
                    const uint32_t t6 = lds_u16(or_code_byte<3>(ub, ml)), t7 = lds_u16(or_code_byte<3>(ub, mh));
                    const u2v b0 = {t0 | (t1 << 16), t2 | (t3 << 16)};
                    const u2v b1 = {t4 | (t5 << 16), t6 | (t7 << 16)};
#pragma unroll
                    for (int p = 0; p < BQ; p++) {
                        acc[u][p] = __builtin_amdgcn_mfma_f32_4x4x4f16(x0[p], __builtin_bit_cast(h4q, b0), acc[u][p], 0, 0, 0);
                        acc[u][p] = __builtin_amdgcn_mfma_f32_4x4x4f16(x1[p], __builtin_bit_cast(h4q, b1), acc[u][p], 0, 0, 0);
                    }
                }
            }
        }
        wave_sync_lds();   // the next group rewrites the tables
        // add the 16 block sums: v[(u * BQ + p) * 4 + i] (token 4p + i, row
        // 4u + j), halves exchanged across lane bits 5 and 4, then butterflies
        // over bits 3, 2
        constexpr int V = 4 * Q * BQ;
        float v[V];
#pragma unroll
        for (int u = 0; u < Q; u++)
#pragma unroll
            for (int p = 0; p < BQ; p++)
#pragma unroll
                for (int i = 0; i < 4; i++) v[(u * BQ + p) * 4 + i] = acc[u][p][i];
#pragma unroll
        for (int m = 0; m < V / 2; m++) v[m] = half_swap_add<32>(v[m], v[m + V / 2]);
#pragma unroll
        for (int m = 0; m < V / 4; m++) v[m] = half_swap_add<16>(v[m], v[m + V / 4]);
#pragma unroll
        for (int m = 0; m < V / 4; m++) {
            v[m] += __shfl_xor(v[m], 8);
            v[m] += __shfl_xor(v[m], 4);
        }
        if ((lane & 12) == 0) {
            const int base = ((lane & 32) ? V / 2 : 0) + ((lane & 16) ? V / 4 : 0);
#pragma unroll
            for (int m = 0; m < V / 4; m++) {
                const int idx = base + m, u = idx / (4 * BQ), p = (idx / 4) % BQ, i = idx % 4;
                const int64_t row = row0 + 4 * u + j;
                const int b = 4 * p + i;
                if (row < N && b < B) y[(size_t)b * N + row] = v[m];
            }
        }
    }
}

template <int Q, int KC, int BQ = 1>
static hipError_t launch_km4_quad_q(const uint8_t *codes, const void *plane, int64_t N, const void *x, int B,
                                    float *y, hipStream_t st, uint64_t *hdr) {
    constexpr int K = 512 * KC;
    const size_t lds = (size_t)4 * BQ * quad_x_row(K) * 2 + (size_t)kQuadWaves * Q * 128;
    if (lds > 64 * 1024) {
        // K = 4096 with two token quads: 77 KiB, two workgroups still fit a CU's 160 KiB
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mv_km4_quad<Q, KC, BQ>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t groups = (N + 4 * Q - 1) / (4 * Q);
    const int64_t want = (groups + kQuadWaves - 1) / kQuadWaves;
    const int64_t cap = 2 * (int64_t)device_cu_count();   // two workgroups per CU stay resident
    const int grid = (int)(want < cap ? want : cap);
    hipLaunchKernelGGL((mv_km4_quad<Q, KC, BQ>), dim3(grid), dim3(64 * kQuadWaves), lds, st, codes,
                       reinterpret_cast<const uint16_t *>(plane), N, reinterpret_cast<const _Float16 *>(x), B, y, hdr);
    return hipGetLastError();
}

// The scale formats (int4, affine int4) on the same 4x4x4 blocks, batch 3-8:
// the codes decode by arithmetic (decode8: magic-number fp16, no lookups), x
// is staged in the decoder's element order, every 32-code chunk (one block)
// is accumulated by its own MFMA chain and added into the fp32 total with the
// block scale (affine int4: plus bias x the block's x sum, from an LDS table
// [chunk][token]). Batch 5-8 takes two token quads (BQ = 2: two MFMAs per
// step on one decoded B operand). Measured on MI355X (HIP graphs,
// 248320 x 2048): int4 B = 4 / 8 55.9 / 61.2 us against 63.5 / 64.5 us for
// mv_mfma; affine int4 58.7 / 65.5 against 78.6 / 81.3. fp4 gained nothing
// (53.4 against 53.0 us at B = 4, slower at B = 8) and keeps mv_mfma.
template <int FMT, int Q, int KC, int BQ>
__global__ __launch_bounds__(64 * kQuadWaves) void mv_quad_scaled(const uint8_t *__restrict__ codes,
                                                                  const void *__restrict__ plane, int64_t N,
                                                                  const _Float16 *__restrict__ x, int B,
                                                                  float *__restrict__ y, uint64_t *__restrict__ hdr) {
    constexpr int K = 512 * KC, CPR = K / 32, ROWS = 4 * Q, NT = 4 * BQ, XROW = quad_x_row(K);
    constexpr bool AFF = (FMT == INT4AFF);
    static_assert(FMT == INT4 || FMT == INT4AFF, "scale formats with 4-bit codes");
    extern __shared__ __align__(16) uint8_t qlds[];
    // fused argmax: the first workgroup zeroes the reduction header
    if (hdr != nullptr && blockIdx.x == 0 && threadIdx.x < kArgmaxHeader) hdr[threadIdx.x] = 0;
    _Float16 *xs = reinterpret_cast<_Float16 *>(qlds);
    float *xsum = reinterpret_cast<float *>(qlds + NT * XROW * 2);   // affine int4: [CPR][NT]
    for (int i = threadIdx.x; i < NT * (K / 8); i += 64 * kQuadWaves) {
        const int b = i / (K / 8), g8 = i - b * (K / 8), k = 8 * g8;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);   // tokens >= B read zeros
        if (b < B) v = stage_group<FMT>(x + (size_t)b * K, g8);
        // a chunk starts 72 bytes after the previous one: two 8-byte stores
        uint2 *d = reinterpret_cast<uint2 *>(xs + b * XROW + (k >> 5) * kQuadXChunk + (k & 31));
        d[0] = make_uint2(v.x, v.y);
        d[1] = make_uint2(v.z, v.w);
    }
    if constexpr (AFF) {
        for (int i = threadIdx.x; i < NT * CPR; i += 64 * kQuadWaves) {
            const int b = i / CPR, c = i - b * CPR;
            float sum = 0.f;
            if (b < B) {
                const uint4 *p = reinterpret_cast<const uint4 *>(x + (size_t)b * K + 32 * c);
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const uint4 v = p[u];
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; e++) sum = dot2(as_h2(w4[e]), as_h2(0x3C003C00u), sum);
                }
            }
            xsum[c * NT + b] = sum;
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int blk = lane >> 2, j = lane & 3;
    const uint32_t xa = (uint32_t)(uintptr_t)xs + (uint32_t)((j * XROW + blk * kQuadXChunk) * 2);
    const int64_t ngroups = (N + ROWS - 1) / ROWS;
    for (int64_t g = (int64_t)blockIdx.x * kQuadWaves + wave; g < ngroups; g += (int64_t)gridDim.x * kQuadWaves) {
        const int64_t row0 = g * ROWS;
        // rows past N read row N - 1 and are never stored
        uint4 cw[Q][KC];
        uint32_t sw[Q][KC];   // block scale (affine int4: scale | bias << 16)
#pragma unroll
        for (int u = 0; u < Q; u++) {
            const int64_t r = row0 + 4 * u + j < N ? row0 + 4 * u + j : N - 1;
#pragma unroll
            for (int kc = 0; kc < KC; kc++) {
                const int c = 16 * kc + blk;
                cw[u][kc] = load_stream16(codes + r * (K / 2) + (uint32_t)c * 16u);
                if constexpr (AFF) sw[u][kc] = reinterpret_cast<const uint32_t *>(plane)[r * CPR + c];
                else sw[u][kc] = reinterpret_cast<const uint16_t *>(plane)[r * CPR + c];
            }
        }
        f4 acc[Q][BQ];
#pragma unroll
        for (int u = 0; u < Q; u++)
#pragma unroll
            for (int p = 0; p < BQ; p++) acc[u][p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            f4 ca[Q][BQ];   // this chunk's sums, before the block scale
#pragma unroll
            for (int u = 0; u < Q; u++)
#pragma unroll
                for (int p = 0; p < BQ; p++) ca[u][p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 4; d++) {
                h4q xv[BQ][2];
#pragma unroll
                for (int p = 0; p < BQ; p++)
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        xv[p][h] = lds_h4(xa + (uint32_t)((p * 4 * XROW + 16 * kc * kQuadXChunk + 8 * d + 4 * h) * 2));
#pragma unroll
                for (int u = 0; u < Q; u++) {
                    const uint32_t w = (d == 0) ? cw[u][kc].x : (d == 1) ? cw[u][kc].y : (d == 2) ? cw[u][kc].z : cw[u][kc].w;
                    typedef uint32_t u4q __attribute__((ext_vector_type(4)));
                    const u4q dv = __builtin_bit_cast(u4q, decode8<FMT>(w, 0u));
                    const u2v b0 = {dv[0], dv[1]}, b1 = {dv[2], dv[3]};
#pragma unroll
                    for (int p = 0; p < BQ; p++) {
                        ca[u][p] = __builtin_amdgcn_mfma_f32_4x4x4f16(xv[p][0], __builtin_bit_cast(h4q, b0), ca[u][p], 0, 0, 0);
                        ca[u][p] = __builtin_amdgcn_mfma_f32_4x4x4f16(xv[p][1], __builtin_bit_cast(h4q, b1), ca[u][p], 0, 0, 0);
                    }
                }
            }
            const int c = 16 * kc + blk;
#pragma unroll
            for (int u = 0; u < Q; u++) {
                const float scl = f16_bits_to_f32((uint16_t)(sw[u][kc] & 0xFFFFu));
#pragma unroll
                for (int p = 0; p < BQ; p++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[u][p][i] = __builtin_fmaf(ca[u][p][i], scl, acc[u][p][i]);
                    if constexpr (AFF) {
                        const float bia = f16_bits_to_f32((uint16_t)(sw[u][kc] >> 16));
                        const f4 xsm = *reinterpret_cast<const f4 *>(xsum + c * NT + 4 * p);
#pragma unroll
                        for (int i = 0; i < 4; i++) acc[u][p][i] = __builtin_fmaf(xsm[i], bia, acc[u][p][i]);
                    }
                }
            }
        }
        // add the 16 block sums: v[(u * BQ + p) * 4 + i] (token 4p + i, row 4u + j)
        constexpr int V = Q * BQ * 4;
        float v[V];
#pragma unroll
        for (int u = 0; u < Q; u++)
#pragma unroll
            for (int p = 0; p < BQ; p++)
#pragma unroll
                for (int i = 0; i < 4; i++) v[(u * BQ + p) * 4 + i] = acc[u][p][i];
#pragma unroll
        for (int m = 0; m < V / 2; m++) v[m] = half_swap_add<32>(v[m], v[m + V / 2]);
#pragma unroll
        for (int m = 0; m < V / 4; m++) v[m] = half_swap_add<16>(v[m], v[m + V / 4]);
#pragma unroll
        for (int m = 0; m < V / 4; m++) {
            v[m] += __shfl_xor(v[m], 8);
            v[m] += __shfl_xor(v[m], 4);
        }
        if ((lane & 12) == 0) {
            const int base = ((lane & 32) ? V / 2 : 0) + ((lane & 16) ? V / 4 : 0);
#pragma unroll
            for (int m = 0; m < V / 4; m++) {
                const int idx = base + m, u = idx / (4 * BQ), p = (idx / 4) % BQ, i = idx % 4;
                const int64_t row = row0 + 4 * u + j;
                const int b = 4 * p + i;
                if (row < N && b < B) y[(size_t)b * N + row] = v[m];
            }
        }
    }
}

template <int FMT, int Q, int KC, int BQ>
static hipError_t launch_quad_scaled_q(const uint8_t *codes, const void *plane, int64_t N, const void *x, int B,
                                       float *y, hipStream_t st, uint64_t *hdr) {
    constexpr int K = 512 * KC, NT = 4 * BQ;
    const size_t lds = (size_t)NT * quad_x_row(K) * 2 + (FMT == INT4AFF ? (size_t)NT * (K / 32) * 4 : 0);
    const int64_t groups = (N + 4 * Q - 1) / (4 * Q);
    const int64_t want = (groups + kQuadWaves - 1) / kQuadWaves;
    const int64_t cap = 2 * (int64_t)device_cu_count();   // two workgroups per CU stay resident
    const int grid = (int)(want < cap ? want : cap);
    if (lds > 64 * 1024) {
        // K = 4096 with two token quads: 74 KiB, two workgroups still fit a CU's 160 KiB
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mv_quad_scaled<FMT, Q, KC, BQ>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((mv_quad_scaled<FMT, Q, KC, BQ>), dim3(grid), dim3(64 * kQuadWaves), lds, st, codes, plane, N,
                       reinterpret_cast<const _Float16 *>(x), B, y, hdr);
    return hipGetLastError();
}

// One token quad up to B = 4, two above. Row quads per wave by size, so the
// grid fills the CUs: one below 32768 rows (below 65536 at B <= 4), two above
// (one at K = 4096, keeping 32 code registers per quad). Measured (HIP graphs,
// K = 2048): int4 B = 3 at 16384 / 24576 / 49152 rows 6.05 / 7.40 / 12.55 us
// with one quad against 6.97 / 8.81 / 13.44 with two; B = 8 at 49152 rows
// 16.90 against 15.37; at 8192 rows two quads leave half the CUs idle.
template <int FMT, int KC>
static hipError_t launch_quad_scaled_k(const uint8_t *codes, const void *plane, int64_t N, const void *x, int B,
                                       float *y, hipStream_t st, uint64_t *hdr) {
    const bool two_tok = B > 4;
    const bool two_rows = KC < 8 && N >= (two_tok ? 32768 : 65536);
    if (two_tok) return two_rows ? launch_quad_scaled_q<FMT, (KC < 8 ? 2 : 1), KC, 2>(codes, plane, N, x, B, y, st, hdr)
                                 : launch_quad_scaled_q<FMT, 1, KC, 2>(codes, plane, N, x, B, y, st, hdr);
    return two_rows ? launch_quad_scaled_q<FMT, (KC < 8 ? 2 : 1), KC, 1>(codes, plane, N, x, B, y, st, hdr)
                    : launch_quad_scaled_q<FMT, 1, KC, 1>(codes, plane, N, x, B, y, st, hdr);
}
template <int FMT>
static hipError_t launch_quad_scaled(const uint8_t *codes, const void *plane, int64_t N, int64_t K, const void *x,
                                     int B, float *y, hipStream_t st, uint64_t *hdr) {
    switch (K) {
    case 512: return launch_quad_scaled_k<FMT, 1>(codes, plane, N, x, B, y, st, hdr);
    case 1024: return launch_quad_scaled_k<FMT, 2>(codes, plane, N, x, B, y, st, hdr);
    case 2048: return launch_quad_scaled_k<FMT, 4>(codes, plane, N, x, B, y, st, hdr);
    default:
        if constexpr (FMT == INT4) return launch_quad_scaled_k<FMT, 8>(codes, plane, N, x, B, y, st, hdr);
        return hipErrorInvalidValue;
    }
}

// Batch 2 too from 16384 rows (int4) and 32768 (affine int4): against the
// dot2 kernel, int4 16384 / 248320 x 2048: 6.8 / 52.3 us against 7.3 / 56.5;
// affine int4 32768 / 248320: 9.8 / 57.1 against 11.7 / 61.9, but 7.6 against
// 6.4 at 16384.
// Batch 3-8 from 8192 rows (affine int4 at B >= 5 from 4096, where the
// alternative is the register-x dot2 kernel: 5.8 against 7.2 us at B = 8);
// against the x-staged dot2 kernel at 8192 x 2048: int4 B = 4 / 8 4.6 / 5.4 us
// against 5.2 / 7.6, affine int4 4.9 / 6.2 against 6.1 / 7.7; at 4096 rows
// the dot2 kernels are as fast or faster.
static bool quad_scaled_takes(int fmt, int64_t N, int64_t K, int B) {
    if (B < 2 || B > 8) return false;
    if (B == 2 && N < (fmt == INT4 ? 16384 : 32768)) return false;
    if (B >= 3 && N < ((fmt == INT4AFF && B >= 5) ? 4096 : 8192)) return false;
    if (fmt == INT4) return K == 512 || K == 1024 || K == 2048 || K == 4096;
    if (fmt == INT4AFF) return K == 512 || K == 1024 || K == 2048;
    return false;
}

// from 8192 rows: 8192 x 2048 at B = 4 5.8 us against 7.1 for the dot2 kernel
// (4096 rows: 5.2 against 4.8). Batch 5-8 runs two token quads: against the
// 16 x 16 x 32 register-table kernel at B = 8, 8192 / 65536 / 124160 rows
// 7.1 / 21.0 / 37.7 us against 9.3 / 23.4 / 41.1, the 248320-row head 77.2
// against 76.6 (72-77 against 75-77 in earlier runs).
static bool km4_quad_takes(int64_t N, int64_t K, int B) {
    return B >= 3 && B <= 8 && N >= 8192 && (K == 512 || K == 1024 || K == 2048 || K == 4096);
}

// Quads per wave: four on the tallest heads, two from 32768 rows, one below
// (248320 x 2048 at B = 4: 60.3 against 63.5 us with two; 32768 rows: 11.7
// against 13.8 us with four; 16384 / 24576 rows at B = 3: 7.5 / 9.0 us with
// one against 8.6 / 10.9 with two); at most 16 code registers x 4 per lane.
template <int KC>
static hipError_t launch_km4_quad_k(const uint8_t *codes, const void *plane, int64_t N, const void *x, int B,
                                    float *y, hipStream_t st, uint64_t *hdr) {
    constexpr int QT = (KC < 8) ? 4 : 2, QM = (KC < 8) ? 2 : 1;
    if (B > 4) {
        // two token quads: two row quads from 32768 rows (at B = 8 on the
        // 248320-row head four measured 76 against 72 us), one below
        if (N >= 32768) return launch_km4_quad_q<2, KC, 2>(codes, plane, N, x, B, y, st, hdr);
        return launch_km4_quad_q<1, KC, 2>(codes, plane, N, x, B, y, st, hdr);
    }
    if (N >= 196608) return launch_km4_quad_q<QT, KC>(codes, plane, N, x, B, y, st, hdr);
    if (N >= 32768) return launch_km4_quad_q<QM, KC>(codes, plane, N, x, B, y, st, hdr);
    return launch_km4_quad_q<1, KC>(codes, plane, N, x, B, y, st, hdr);
}
static hipError_t launch_km4_quad(const uint8_t *codes, const void *plane, int64_t N, int64_t K, const void *x,
                                  int B, float *y, hipStream_t st, uint64_t *hdr) {
    switch (K) {
    case 512: return launch_km4_quad_k<1>(codes, plane, N, x, B, y, st, hdr);
    case 1024: return launch_km4_quad_k<2>(codes, plane, N, x, B, y, st, hdr);
    case 2048: return launch_km4_quad_k<4>(codes, plane, N, x, B, y, st, hdr);
    default: return launch_km4_quad_k<8>(codes, plane, N, x, B, y, st, hdr);
    }
}

template <int FMT>
static size_t mfma_lds_bytes(int64_t K, int B) {
    return (size_t)B * (size_t)(K + 8) * 2 + kZeroLds + (size_t)xsum_lds_bytes<FMT>((int)K) +
           (size_t)kMfmaWaves * wave_lds_bytes<FMT, kLdsCodes>((int)K);
}

// The batched matrix-core path takes int4, affine int4 (K <= 2048), fp4, int8,
// km4 and int8 k-means, fp16 x, 3 <= B <= 8, whole load steps (K % 512 == 0,
// int8 and int8 k-means K % 256 == 0), K <= 4096, N >= 16, a 16-byte aligned
// scale plane, and staging that fits in 64 KiB of LDS (affine int4: 80 KiB,
// two workgroups per CU).
static bool mfma_eligible(int fmt, const void *plane, int64_t N, int64_t K, int B) {
    // a group's scales (tables) are read as 16-byte pieces
    if (reinterpret_cast<uintptr_t>(plane) % 16 != 0) return false;
    // the 4x4x4 kernels have their own size rules and stage x alone (at most
    // 74 KiB, two workgroups per CU)
    if ((fmt == KM4 && km4_quad_takes(N, K, B)) || quad_scaled_takes(fmt, N, K, B)) return true;
    if (B < 3 || B > 8 || N < 16) return false;
    // below 16384 rows the dot2 path is as fast at B = 3, 4 (fp4 4096 x 2048:
    // 6.8 us against 7.4 us); from B = 5 the matrix cores win at any size
    if (B <= 4 && N < 16384) return false;
    // up to 4096 rows of one 1024-byte chunk per lane (4-bit K 1025..2048,
    // int8 two chunks) the dot2 kernel is faster at B = 5-8 too (HIP graphs,
    // B = 5 / 8: fp4 4096 x 2048 5.9 / 6.2 us against 7.0 / 7.6; int4 7.0 /
    // 7.4 against 8.3 / 8.9; km4 5.9 / 6.4 against 8.6 / 9.2; int8 k-means
    // 6.4 / 6.5 against 12.9 / 13.5)
    if (N <= 4096 && K > 1024 && K <= 2048) return false;
    // the dot2 kernel with x staged in LDS (int4, fp4, int8 at K = 2048) is
    // faster up to 8192 rows too (8192 x 2048 at B = 8, HIP graphs: fp4 6.7
    // against 7.8 us, int4 7.4 against 8.9, int8 8.2 against 11.3; at 16384
    // rows the matrix cores win: fp4 8.5 against 11.2)
    if (N <= 8192 && B >= 5 && K == 2048 && (fmt == INT4 || fmt == FP4 || fmt == INT8)) return false;
    if (fmt == INT4AFF && K > 2048) return false;   // its scale + bias stretch fits four pieces per lane
    if (K % ((fmt == INT8 || fmt == INT8KM) ? 256 : 512) != 0 || K > 4096) return false;
    size_t lds = (fmt == INT4) ? mfma_lds_bytes<INT4>(K, B)
                 : (fmt == INT4AFF) ? mfma_lds_bytes<INT4AFF>(K, B)
                 : (fmt == FP4) ? mfma_lds_bytes<FP4>(K, B)
                 : (fmt == INT8) ? mfma_lds_bytes<INT8>(K, B)
                 : (fmt == INT8KM) ? mfma_lds_bytes<INT8KM>(K, B) : mfma_lds_bytes<KM4>(K, B);
    return lds <= (fmt == INT4AFF ? 80 : 64) * 1024;
}

template <int FMT, int SP, int RG>
static hipError_t launch_mfma_rg(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                                 float *y, hipStream_t st, uint64_t *hdr) {
    constexpr int D = 2;
    const int64_t rows_wg = (int64_t)kMfmaWaves * RG * 16;
    const int64_t grid = (N + rows_wg - 1) / rows_wg;
    const size_t lds = mfma_lds_bytes<FMT>(K, B);
    if (lds > 64 * 1024) {
        // two workgroups still fit a CU's 160 KiB; allow the larger dynamic allocation
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mv_mfma<FMT, RG, SP, D, kLdsCodes>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((mv_mfma<FMT, RG, SP, D, kLdsCodes>), dim3((unsigned)grid), dim3(64 * kMfmaWaves), lds, st,
                       codes, plane, N, K, reinterpret_cast<const _Float16 *>(x), B, y, hdr);
    return hipGetLastError();
}

// Row groups per wave: about 512 workgroups (two per CU, the residency the
// LDS staging allows) whatever N; measured on MI355X at B = 4 and 8: 4096 to
// 32768 rows are fastest with one group per wave, 65536 with two, the
// 248320-row lm_head with eight.
template <int FMT, int SP>
static hipError_t launch_mfma_sp(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                                 float *y, hipStream_t st, uint64_t *hdr) {
    const int64_t per_rg1 = (int64_t)kMfmaWaves * 16 * 512;   // rows that give 512 workgroups at RG = 1
    if (N >= 6 * per_rg1) return launch_mfma_rg<FMT, SP, 8>(codes, plane, N, K, x, B, y, st, hdr);
    if (N >= 3 * per_rg1) return launch_mfma_rg<FMT, SP, 4>(codes, plane, N, K, x, B, y, st, hdr);
    if (N >= (3 * per_rg1) / 2) return launch_mfma_rg<FMT, SP, 2>(codes, plane, N, K, x, B, y, st, hdr);
    return launch_mfma_rg<FMT, SP, 1>(codes, plane, N, K, x, B, y, st, hdr);
}

template <int FMT>
static hipError_t launch_mfma_fmt(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                                  float *y, hipStream_t st, uint64_t *hdr) {
    const int sp = scale_pieces<FMT>(K);
    if (sp <= 1) return launch_mfma_sp<FMT, 1>(codes, plane, N, K, x, B, y, st, hdr);
    if (sp <= 2) return launch_mfma_sp<FMT, 2>(codes, plane, N, K, x, B, y, st, hdr);
    return launch_mfma_sp<FMT, 4>(codes, plane, N, K, x, B, y, st, hdr);
}

hipError_t launch_matvec_mfma(int fmt, const uint8_t *codes, const void *plane, int64_t N, int64_t K, const void *x,
                              int B, float *y, hipStream_t st, bool *handled, uint64_t *hdr) {
    *handled = mfma_eligible(fmt, plane, N, K, B);
    if (!*handled) return hipSuccess;
    if (fmt == KM4 && km4_quad_takes(N, K, B)) return launch_km4_quad(codes, plane, N, K, x, B, y, st, hdr);
    if (quad_scaled_takes(fmt, N, K, B))
        return fmt == INT4 ? launch_quad_scaled<INT4>(codes, plane, N, K, x, B, y, st, hdr)
                           : launch_quad_scaled<INT4AFF>(codes, plane, N, K, x, B, y, st, hdr);
    switch (fmt) {
    case INT4: return launch_mfma_fmt<INT4>(codes, plane, N, (int)K, x, B, y, st, hdr);
    case INT4AFF: return launch_mfma_fmt<INT4AFF>(codes, plane, N, (int)K, x, B, y, st, hdr);
    case FP4: return launch_mfma_fmt<FP4>(codes, plane, N, (int)K, x, B, y, st, hdr);
    case INT8: return launch_mfma_fmt<INT8>(codes, plane, N, (int)K, x, B, y, st, hdr);
    case INT8KM: return launch_mfma_fmt<INT8KM>(codes, plane, N, (int)K, x, B, y, st, hdr);
    default: return launch_mfma_fmt<KM4>(codes, plane, N, (int)K, x, B, y, st, hdr);
    }
}

}  // namespace qmv
