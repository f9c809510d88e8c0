// Mixture-of-experts decode: top-k routing and the routed-expert gather
// matvec ("Stream D - Quantization (FP4 + QAT-int4)...", section 1: the
// gather_qmm kernels over expert slabs blocked along K; "Dense-path int4km
// coverage + flagship Qwen3.6-35B...", section 1: only the routed experts'
// weights are read, avoiding the all-experts over-read).
//
// gfx950 design. Decode touches at most T*topk experts and is latency-bound
// at small T, so the layer is two launches:
//  1. gate/up + SwiGLU, expert-major: each workgroup takes one (unique
//     expert, row tile). The unique-expert list is rebuilt in the workgroup
//     from the T*topk ids (an LDS bitmap and wave ballots), so a chosen
//     expert's weights are read once however many tokens chose it. For a
//     single token the routing is fused in: every workgroup routes the token
//     itself (DPP reductions over registers) and workgroup (0,0) publishes
//     ids and weights for launch 2; for more tokens a small routing launch
//     runs first.
//  2. down + weighted combine, token-major: each workgroup takes one (token,
//     row tile) and walks the token's slots in slot order, accumulating
//     w * (W_down[e] h) in registers. No partial buffer, no combine launch,
//     and the sum order is fixed, so results are deterministic. An expert
//     chosen by several tokens is re-read from L2 / Infinity Cache.
#include "qmv_device.h"
#include "qmv_launch.h"

namespace qmv {

enum Epi { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_COMBINE = 2 };

// ---------------------------------------------------------------------------
// routing
// ---------------------------------------------------------------------------
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// max over the wave, returned in every lane (DPP within 16-lane rows, then
// the four row results read into scalars)
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Top-k of one token's E logits, largest first, equal logits in increasing
// expert order; softmax over the selected logits. Lane j < topk returns the
// j-th id and weight. Lane l keeps logits l, l + 64, ... in registers.
template <int PER_LANE>
__device__ __forceinline__ void route_token(const float *__restrict__ l, int E, int topk, int lane, int &out_id,
                                            float &out_w) {
    float v[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; i++) {
        int e = lane + 64 * i;
        v[i] = l[e < E ? e : 0];
    }
    uint64_t taken = 0;
    int my_i = 0;
    float my_v = 0.f;
    for (int j = 0; j < topk; j++) {
        float best = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < PER_LANE; i++)
            if (lane + 64 * i < E && !((taken >> i) & 1ull)) best = fmaxf(best, v[i]);
        const float m = wave_max(best);
        // the lowest untaken expert id holding the maximum: ids lane + 64 i,
        // so the first slot i with a holder, then its lowest lane (one wave
        // ballot per slot, scalar find-first-set)
        int sel = 0x7fffffff;
#pragma unroll
        for (int i = PER_LANE - 1; i >= 0; i--) {
            const uint64_t b = __ballot(lane + 64 * i < E && !((taken >> i) & 1ull) && v[i] == m);
            if (b != 0ull) sel = 64 * i + __builtin_ctzll(b);
        }
        if (sel == 0x7fffffff) {
            // only NaN logits left untaken: the lowest untaken id (NaN ranks
            // below every number), so ids stay valid expert indices
#pragma unroll
            for (int i = PER_LANE - 1; i >= 0; i--) {
                const uint64_t b = __ballot(lane + 64 * i < E && !((taken >> i) & 1ull));
                if (b != 0ull) sel = 64 * i + __builtin_ctzll(b);
            }
        }
        if ((sel & 63) == lane) taken |= 1ull << (sel >> 6);
        if (lane == j) {
            my_i = sel;
            my_v = m;
        }
    }
    const float vmax = readlane_f(my_v, 0);
    const float p = lane < topk ? expf(my_v - vmax) : 0.f;
    const float z = wave_sum(p);
    out_id = my_i;
    out_w = p / z;
}

constexpr int route_per_lane(int E) { return E <= 256 ? 4 : (E <= 1024 ? 16 : 64); }

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int T, int E, int topk,
                                                    int32_t *__restrict__ ids, float *__restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int id;
    float w;
    route_token<PER_LANE>(logits + (int64_t)t * E, E, topk, lane, id, w);
    if (lane < topk) {
        ids[(int64_t)t * topk + lane] = id;
        weights[(int64_t)t * topk + lane] = w;
    }
}

hipError_t launch_moe_route(const float *logits, int T, int E, int topk, int32_t *ids, float *weights,
                            hipStream_t st) {
    const int pl = route_per_lane(E);
    if (pl == 4)
        hipLaunchKernelGGL(route_kernel<4>, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, topk, ids, weights);
    else if (pl == 16)
        hipLaunchKernelGGL(route_kernel<16>, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, topk, ids, weights);
    else
        hipLaunchKernelGGL(route_kernel<64>, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, topk, ids, weights);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ float plane_scale(const void *plane, int64_t row, int nb, int c) {
    if constexpr (FMT == INT4 || FMT == INT8) {
        int blk = (FMT == INT8) ? c / 2 : c;
        return f16_bits_to_f32(reinterpret_cast<const uint16_t *>(plane)[row * nb + blk]);
    } else if constexpr (FMT == FP4) {
        return e8m0_to_f32(reinterpret_cast<const uint8_t *>(plane)[row * nb + c]);
    } else if constexpr (FMT == INT4AFF) {
        return f16_bits_to_f32((uint16_t)(reinterpret_cast<const uint32_t *>(plane)[row * nb + c] & 0xFFFFu));
    } else {
        return 1.f;
    }
}

// affine int4: the block's bias (it multiplies the block's x sum)
template <int FMT>
__device__ __forceinline__ float plane_bias(const void *plane, int64_t row, int nb, int c) {
    if constexpr (FMT == INT4AFF)
        return f16_bits_to_f32((uint16_t)(reinterpret_cast<const uint32_t *>(plane)[row * nb + c] >> 16));
    else
        return 0.f;
}

template <int FMT>
__device__ __forceinline__ int64_t code_row_bytes(int K) { return (FMT == INT8 || FMT == INT8KM) ? K : K / 2; }

// expert e's code and plane slabs
template <int FMT>
__device__ __forceinline__ void expert_slabs(const uint8_t *codes, const void *plane, int64_t e, int64_t N, int K,
                                             const uint8_t *&codes_e, const void *&plane_e) {
    codes_e = codes + e * N * code_row_bytes<FMT>(K);
    if constexpr (FMT == FP4)
        plane_e = reinterpret_cast<const uint8_t *>(plane) + e * N * (K / 32);
    else if constexpr (FMT == KM4)
        plane_e = reinterpret_cast<const uint16_t *>(plane) + e * N * 16;
    else if constexpr (FMT == INT4AFF)
        plane_e = reinterpret_cast<const uint32_t *>(plane) + e * N * (K / 32);
    else if constexpr (FMT == INT8KM)
        plane_e = reinterpret_cast<const uint16_t *>(plane) + e * (N / 32) * 256;   // N % 32 == 0
    else
        plane_e = reinterpret_cast<const uint16_t *>(plane) + e * N * (K / 32);
}

template <int FMT>
__device__ __forceinline__ float chunk_dot(uint4 cw, const uint32_t (&xw)[ChunkTraits<FMT>::kXWords],
                                           const _Float16 *lut) {
    if constexpr (FMT == INT4) return chunk_dot_int4(cw, xw);
    else if constexpr (FMT == INT4AFF) return chunk_dot_int4<true>(cw, xw);
    else if constexpr (FMT == FP4) return chunk_dot_fp4(cw, xw);
    else if constexpr (FMT == INT8) return chunk_dot_int8(cw, xw);
    else if constexpr (FMT == INT8KM) return chunk_dot_int8km(cw, lut, xw);
    else return chunk_dot_km4(cw, lut, xw);
}

__device__ __forceinline__ void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct GatherArgs {
    const uint8_t *codes;
    const void *plane;
    int E;
    int64_t N;          // rows per expert
    int K;
    const _Float16 *x;
    int x_per_slot;
    int T, topk;
    const int32_t *ids;
    const float *weights;
    const float *logits;  // fused routing: logits [T][E]; ids/weights are then outputs
    int32_t *ids_out;
    float *weights_out;
    void *out;
    int64_t out_rows;   // logical rows per pair (N, or N/2 for SWIGLU)
    int tile_rows;      // logical rows per workgroup
};

// ---------------------------------------------------------------------------
// expert-major gather (NONE, SWIGLU)
// ---------------------------------------------------------------------------
// One pass over the workgroup's row tile for PB token slots (pairs).
// R row groups per wave iteration; with SWIGLU the first R/2 groups are gate
// rows and the last R/2 the matching up rows. Loads are unconditional (rows
// clamped into the tile, chunks past the row end read chunk 0 against a zero
// x slice) and stream past the caches. An expert chosen by more than two
// tokens is read once per pass; keeping its codes in registers across passes
// instead costs more registers (fewer resident waves) than it saves, since
// most chosen experts have one or two slots in a decode batch.
template <int FMT, int PB, int LPR, int CPL, int R, int EPI>
__device__ __forceinline__ void gather_pass(const GatherArgs &a, const uint8_t *__restrict__ codes_e,
                                            const void *__restrict__ plane_e, const int *pairs,
                                            _Float16 *lut_w) {
    constexpr int RPW = kWave / LPR;
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    constexpr int G = (EPI == EPI_SWIGLU) ? R / 2 : R;   // logical row groups per iteration
    constexpr int LROWS = G * RPW;                       // logical rows per iteration
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int rsub = lane / LPR;
    const int K = a.K;
    const int cpr = (FMT == INT8 || FMT == INT8KM) ? K / 16 : K / 32;
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)code_row_bytes<FMT>(K);

    constexpr bool AFF = (FMT == INT4AFF);
    constexpr bool KM8 = (FMT == INT8KM);
    uint32_t xr[CPL][PB][XW];
    float xsum[AFF ? CPL : 1][AFF ? PB : 1];
#pragma unroll
    for (int p = 0; p < PB; p++) {
        int pr = pairs[p];
        const _Float16 *xp = a.x + (int64_t)(a.x_per_slot ? pr : pr / a.topk) * K;
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            int c = sub + LPR * j;
            load_x_slice<FMT>(xp, c, c < cpr, xr[j][p]);
            if constexpr (AFF) xsum[j][p] = x_slice_sum<XW>(xr[j][p]);
        }
    }
    const int64_t tile0 = (int64_t)blockIdx.x * a.tile_rows;
    int64_t tile1 = tile0 + a.tile_rows;
    if (tile1 > a.out_rows) tile1 = a.out_rows;
    for (int64_t l0 = tile0 + (int64_t)wave * LROWS; l0 < tile1; l0 += 4 * LROWS) {
        uint4 cw[R][CPL];
        float sc[R][CPL];
        float bi[AFF ? R : 1][AFF ? CPL : 1];
#pragma unroll
        for (int g = 0; g < R; g++) {
            int gl = (EPI == EPI_SWIGLU) ? (g % G) : g;
            int64_t lrow = l0 + gl * RPW + rsub;
            lrow = lrow < tile1 ? lrow : tile1 - 1;
            int64_t prow = (EPI == EPI_SWIGLU && g >= G) ? lrow + a.out_rows : lrow;
            const uint8_t *rp = codes_e + prow * (int64_t)row_bytes;
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                int c = sub + LPR * j;
                int cc = c < cpr ? c : 0;
                cw[g][j] = load_stream16(rp + (uint32_t)cc * 16u);
                sc[g][j] = plane_scale<FMT>(plane_e, prow, nb, cc);
                if constexpr (AFF) bi[g][j] = plane_bias<FMT>(plane_e, prow, nb, cc);
            }
        }
        if constexpr (FMT == KM4) {
            const uint32_t *lsrc = reinterpret_cast<const uint32_t *>(plane_e);
            uint32_t *ldst = reinterpret_cast<uint32_t *>(lut_w);
            for (int i = lane; i < R * RPW * 8; i += kWave) {
                int g = i / (RPW * 8), rs = (i / 8) % RPW;
                int gl = (EPI == EPI_SWIGLU) ? (g % G) : g;
                int64_t lrow = l0 + gl * RPW + rs;
                lrow = lrow < tile1 ? lrow : tile1 - 1;
                int64_t pr = (EPI == EPI_SWIGLU && g >= G) ? lrow + a.out_rows : lrow;
                ldst[i] = lsrc[pr * 8 + (i % 8)];
            }
            wave_fence();
        } else if constexpr (KM8) {
            // one 256-entry table per row group: its RPW rows are aligned and
            // lie in one group of 32 (the first row, clamped, names it)
            const uint32_t *lsrc = reinterpret_cast<const uint32_t *>(plane_e);
            uint32_t *ldst = reinterpret_cast<uint32_t *>(lut_w);
            uint32_t tv[R][2];
#pragma unroll
            for (int g = 0; g < R; g++) {
                int gl = (EPI == EPI_SWIGLU) ? (g % G) : g;
                int64_t lrow = l0 + gl * RPW;
                lrow = lrow < tile1 ? lrow : tile1 - 1;
                int64_t pr = (EPI == EPI_SWIGLU && g >= G) ? lrow + a.out_rows : lrow;
#pragma unroll
                for (int q = 0; q < 2; q++) tv[g][q] = lsrc[(pr / 32) * 128 + q * kWave + lane];
            }
#pragma unroll
            for (int g = 0; g < R; g++)
#pragma unroll
                for (int q = 0; q < 2; q++) ldst[g * 128 + q * kWave + lane] = tv[g][q];
            wave_fence();
        }
        float acc[R * PB];
#pragma unroll
        for (int g = 0; g < R; g++)
#pragma unroll
            for (int p = 0; p < PB; p++) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    float d = chunk_dot<FMT>(cw[g][j], xr[j][p], KM8 ? lut_w + g * 256 : lut_w + (g * RPW + rsub) * 16);
                    s = (FMT == KM4 || KM8) ? s + d : __builtin_fmaf(d, sc[g][j], s);
                    if constexpr (AFF) s = __builtin_fmaf(xsum[j][p], bi[g][j], s);
                }
                acc[g * PB + p] = s;
            }
        if constexpr (FMT == KM4 || KM8) wave_fence();   // the next iteration rewrites the tables
        if constexpr (EPI == EPI_SWIGLU) {
            // full reduction: every lane gets every row sum, so each gate sum
            // meets its up sum (group g + G) in the same lane
#pragma unroll
            for (int q = 0; q < R * PB; q++) {
                float v = row16_sum(acc[q]);
                if constexpr (LPR >= 32) v = half_swap_add<16>(v, v);
                if constexpr (LPR == 64) v = half_swap_add<32>(v, v);
                acc[q] = v;
            }
            if (sub == 0) {
#pragma unroll
                for (int g = 0; g < G; g++) {
                    int64_t lrow = l0 + g * RPW + rsub;
                    if (lrow >= tile1) continue;
#pragma unroll
                    for (int p = 0; p < PB; p++) {
                        float gt = acc[g * PB + p], up = acc[(g + G) * PB + p];
                        float h = gt / (1.0f + expf(-gt)) * up;
                        reinterpret_cast<_Float16 *>(a.out)[(int64_t)pairs[p] * a.out_rows + lrow] = (_Float16)h;
                    }
                }
            }
        } else {
            using Red = GroupReduce<R * PB, LPR>;
            Red::run(acc, lane);
            if (Red::writer(lane)) {
                const int base = Red::base(lane);
#pragma unroll
                for (int j = 0; j < Red::live; j++) {
                    int idx = base + j, g = idx / PB, p = idx % PB;
                    int64_t lrow = l0 + g * RPW + rsub;
                    if (lrow < tile1) reinterpret_cast<float *>(a.out)[(int64_t)pairs[p] * a.out_rows + lrow] = acc[j];
                }
            }
        }
    }
}

template <int FMT, int LPR, int CPL, int R, int EPI, bool FUSED_ROUTE, int ROUTE_PL>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    constexpr int RPW = kWave / LPR;
    __shared__ int s_ids[512];
    __shared__ uint32_t s_bits[128];   // one bit per expert id (E <= 4096)
    __shared__ int s_pairs[8];
    __shared__ int s_np;
    __shared__ int s_expert;
    constexpr int LUT_HALVES = (FMT == KM4) ? R * RPW * 16 : (FMT == INT8KM ? R * 256 : 1);   // per wave
    __shared__ _Float16 lut_lds[4 * LUT_HALVES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int npairs = a.T * a.topk;
    const int u = blockIdx.y;
    for (int i = tid; i < 128; i += blockDim.x) s_bits[i] = 0;
    if constexpr (FUSED_ROUTE) {
        // route the tokens here: wave w takes tokens w, w + 4
        const bool publish = blockIdx.x == 0 && blockIdx.y == 0;
        for (int t = tid >> 6; t < a.T; t += 4) {
            int id;
            float w;
            route_token<ROUTE_PL>(a.logits + (int64_t)t * a.E, a.E, a.topk, lane, id, w);
            if (lane < a.topk) {
                s_ids[t * a.topk + lane] = id;
                if (publish) {
                    a.ids_out[t * a.topk + lane] = id;
                    a.weights_out[t * a.topk + lane] = w;
                }
            }
        }
    } else {
        // ids outside [0, E) are clamped into it: no read outside the expert slabs
        for (int i = tid; i < npairs; i += blockDim.x) {
            const int e = a.ids[i];
            s_ids[i] = e < 0 ? 0 : (e < a.E ? e : a.E - 1);
        }
    }
    __syncthreads();
    for (int i = tid; i < npairs; i += blockDim.x) {
        int e = s_ids[i];
        atomicOr(&s_bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    if (tid == 0) {
        // the u-th smallest distinct expert id (u counts from 0)
        int found = -1, before = 0;
        for (int w = 0; w < (a.E + 31) / 32; w++) {
            uint32_t m = s_bits[w];
            int c = __builtin_popcount(m);
            if (u < before + c) {
                for (int k = u - before; k > 0; k--) m &= m - 1;   // drop the lower set bits
                found = 32 * w + __builtin_ctz(m);
                break;
            }
            before += c;
        }
        s_expert = found;
    }
    __syncthreads();
    if (tid < 64) {
        // token slots that chose this expert, in slot order, via wave ballots
        const int e = s_expert;
        int np = 0;
        for (int base = 0; base < npairs && e >= 0; base += 64) {
            int i = base + tid;
            uint64_t m = __ballot(i < npairs && s_ids[i] == e);
            int before = __builtin_popcountll(m & ((1ull << tid) - 1));
            if (((m >> tid) & 1ull) && np + before < 8) s_pairs[np + before] = i;
            np += __builtin_popcountll(m);
        }
        if (tid == 0) s_np = np < 8 ? np : 8;
    }
    __syncthreads();
    const int e = s_expert;
    if (e < 0) return;
    const int np = s_np;
    const uint8_t *codes_e;
    const void *plane_e;
    expert_slabs<FMT>(a.codes, a.plane, e, a.N, a.K, codes_e, plane_e);
    _Float16 *lut_w = lut_lds + (tid >> 6) * LUT_HALVES;
    int p0 = 0;
    for (; p0 + 2 <= np; p0 += 2)
        gather_pass<FMT, 2, LPR, CPL, R, EPI>(a, codes_e, plane_e, s_pairs + p0, lut_w);
    if (p0 < np) gather_pass<FMT, 1, LPR, CPL, R, EPI>(a, codes_e, plane_e, s_pairs + p0, lut_w);
}

// ---------------------------------------------------------------------------
// token-major down projection with the weighted combine fused
//   y[t][n] = sum over slots s (in order) of w[t][s] * (W[ids[t][s]] x_{t,s})[n]
// One wave per workgroup; the wave owns ROWS = R * (64 / LPR) rows of token t.
// The slots are taken in batches of SB: the codes, scales and x slices of
// every slot of a batch are loaded at once, so the wave waits for one memory
// round trip per batch instead of one per slot.
// ---------------------------------------------------------------------------
template <int FMT, int R, int CPL>
constexpr int combine_slot_batch() {
    constexpr int per_slot = 5 * R * CPL + ChunkTraits<FMT>::kXWords * CPL + (FMT == KM4 ? 1 : (FMT == INT8KM ? 2 : 0));
    constexpr int sb = 192 / per_slot;
    return sb < 1 ? 1 : (sb > 8 ? 8 : sb);
}

template <int FMT, int LPR, int CPL, int R, int SB>
__global__ __launch_bounds__(64) void combine_gather_kernel(GatherArgs a) {
    constexpr int RPW = kWave / LPR;
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    constexpr int ROWS = R * RPW;
    // int8km: ROWS divides 32 and row0 is a multiple of ROWS, so the wave's
    // rows share one table per slot
    constexpr bool KM8 = (FMT == INT8KM);
    static_assert(!KM8 || 32 % ROWS == 0, "int8km: a wave's rows within one group");
    __shared__ _Float16 lut_lds[(FMT == KM4) ? SB * ROWS * 16 : (KM8 ? SB * 256 : 1)];
    const int lane = threadIdx.x;
    const int sub = lane % LPR;
    const int rsub = lane / LPR;
    const int t = blockIdx.y;
    const int K = a.K;
    const int cpr = (FMT == INT8 || KM8) ? K / 16 : K / 32;
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)code_row_bytes<FMT>(K);
    const int64_t row0 = (int64_t)blockIdx.x * ROWS;
    if (row0 >= a.N) return;
    const int last = (int)((a.N - 1 - row0) < ROWS - 1 ? (a.N - 1 - row0) : ROWS - 1);

    float acc[R];
#pragma unroll
    for (int g = 0; g < R; g++) acc[g] = 0.f;
    for (int s0 = 0; s0 < a.topk; s0 += SB) {
        constexpr bool AFF = (FMT == INT4AFF);
        uint4 cw[SB][R][CPL];
        float sc[SB][R][CPL];
        float bi[AFF ? SB : 1][AFF ? R : 1][AFF ? CPL : 1];
        float xs[AFF ? SB : 1][AFF ? CPL : 1];
        uint32_t xr[SB][CPL][XW];
        float ws[SB];
        uint32_t lutv[SB][KM8 ? 2 : 1];
#pragma unroll
        for (int b = 0; b < SB; b++) {
            // slots past topk repeat the last one with weight 0
            const int s = s0 + b < a.topk ? s0 + b : a.topk - 1;
            const int e0 = a.ids[t * a.topk + s];
            const int e = e0 < 0 ? 0 : (e0 < a.E ? e0 : a.E - 1);   // clamped, as in the expert-major kernel
            ws[b] = s0 + b < a.topk ? a.weights[t * a.topk + s] : 0.f;
            const uint8_t *codes_e;
            const void *plane_e;
            expert_slabs<FMT>(a.codes, a.plane, e, a.N, K, codes_e, plane_e);
#pragma unroll
            for (int g = 0; g < R; g++) {
                int rr = g * RPW + rsub;
                rr = rr <= last ? rr : last;
                const int64_t row = row0 + rr;
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    int c = sub + LPR * j;
                    int cc = c < cpr ? c : 0;
                    cw[b][g][j] = load_stream16(codes_e + row * (int64_t)row_bytes + (uint32_t)cc * 16u);
                    sc[b][g][j] = plane_scale<FMT>(plane_e, row, nb, cc);
                    if constexpr (AFF) bi[b][g][j] = plane_bias<FMT>(plane_e, row, nb, cc);
                }
            }
            const _Float16 *xp = a.x + (int64_t)(a.x_per_slot ? t * a.topk + s : t) * K;
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                int c = sub + LPR * j;
                load_x_slice<FMT>(xp, c, c < cpr, xr[b][j]);
                if constexpr (AFF) xs[b][j] = x_slice_sum<XW>(xr[b][j]);
            }
            if constexpr (FMT == KM4) {
                int rr = (lane / 8) % ROWS;
                rr = rr <= last ? rr : last;
                lutv[b][0] = reinterpret_cast<const uint32_t *>(plane_e)[(row0 + rr) * 8 + (lane % 8)];
            } else if constexpr (KM8) {
#pragma unroll
                for (int q = 0; q < 2; q++)
                    lutv[b][q] = reinterpret_cast<const uint32_t *>(plane_e)[(row0 / 32) * 128 + q * kWave + lane];
            }
        }
        if constexpr (FMT == KM4) {
#pragma unroll
            for (int b = 0; b < SB; b++)
                if (lane < ROWS * 8) reinterpret_cast<uint32_t *>(lut_lds)[b * ROWS * 8 + lane] = lutv[b][0];
            wave_fence();
        } else if constexpr (KM8) {
#pragma unroll
            for (int b = 0; b < SB; b++)
#pragma unroll
                for (int q = 0; q < 2; q++) reinterpret_cast<uint32_t *>(lut_lds)[b * 128 + q * kWave + lane] = lutv[b][q];
            wave_fence();
        }
#pragma unroll
        for (int b = 0; b < SB; b++)
#pragma unroll
            for (int g = 0; g < R; g++)
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    float d = chunk_dot<FMT>(cw[b][g][j], xr[b][j],
                                             KM8 ? lut_lds + b * 256 : lut_lds + (b * ROWS + g * RPW + rsub) * 16);
                    acc[g] = __builtin_fmaf(d, ws[b] * sc[b][g][j], acc[g]);
                    if constexpr (AFF) acc[g] = __builtin_fmaf(xs[b][j], ws[b] * bi[b][g][j], acc[g]);
                }
        if constexpr (FMT == KM4 || KM8) wave_fence();   // the next batch rewrites the tables
    }
    using Red = GroupReduce<R, LPR>;
    Red::run(acc, lane);
    if (Red::writer(lane)) {
        const int base = Red::base(lane);
#pragma unroll
        for (int j = 0; j < Red::live; j++) {
            int64_t row = row0 + (base + j) * RPW + rsub;
            if (row < a.N) reinterpret_cast<float *>(a.out)[(int64_t)t * a.N + row] = acc[j];
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
size_t gather_workspace_bytes(int, int, int, int64_t, int) { return 0; }

template <int FMT, int LPR, int CPL, int EPI, bool FUSED, int R>
static hipError_t launch_expert_major_r(GatherArgs a, int umax, hipStream_t st) {
    constexpr int RPW = kWave / LPR;
    constexpr int G = (EPI == EPI_SWIGLU) ? R / 2 : R;
    // one iteration per wave: many small workgroups keep every load in flight
    a.tile_rows = 4 * G * RPW;
    int tiles = (int)((a.out_rows + a.tile_rows - 1) / a.tile_rows);
    if constexpr (!FUSED) {
        hipLaunchKernelGGL((gather_kernel<FMT, LPR, CPL, R, EPI, false, 4>), dim3(tiles, umax), dim3(256), 0, st, a);
    } else {
        const int pl = route_per_lane(a.E);
        if (pl == 4)
            hipLaunchKernelGGL((gather_kernel<FMT, LPR, CPL, R, EPI, true, 4>), dim3(tiles, umax), dim3(256), 0, st, a);
        else if (pl == 16)
            hipLaunchKernelGGL((gather_kernel<FMT, LPR, CPL, R, EPI, true, 16>), dim3(tiles, umax), dim3(256), 0, st,
                               a);
        else
            hipLaunchKernelGGL((gather_kernel<FMT, LPR, CPL, R, EPI, true, 64>), dim3(tiles, umax), dim3(256), 0, st,
                               a);
    }
    return hipGetLastError();
}

template <int FMT, int LPR, int CPL, int EPI, bool FUSED>
static hipError_t launch_expert_major(GatherArgs a, int umax, hipStream_t st) {
    // gate and up rows in pairs; fewer rows per iteration on long rows (and
    // for table lookups, which hold more registers) to stay within the
    // register file. Several tokens with one chunk per lane and no tables take
    // 4 gate and 4 up rows per wave (int4 T = 8: 33.5 us against 34.8 us with
    // 2 + 2); one token keeps 2 + 2 (more, smaller waves).
    constexpr int heavy = (FMT == KM4 || FMT == INT8KM) ? CPL + 1 : CPL;
    if constexpr (EPI == EPI_SWIGLU && !FUSED && heavy == 1) {
        if (a.T > 1) return launch_expert_major_r<FMT, LPR, CPL, EPI, FUSED, 8>(a, umax, st);
    }
    constexpr int R = (EPI == EPI_SWIGLU) ? (heavy >= 3 ? 2 : 4) : (heavy >= 3 ? 1 : 2);
    return launch_expert_major_r<FMT, LPR, CPL, EPI, FUSED, R>(a, umax, st);
}

// ---------------------------------------------------------------------------
// Slot-split down projection + combine, topk <= kSplitSlots: a workgroup of
// kSplitSlots waves owns ROWS rows of token t, wave s computes slot s's
// weighted row sums w_s * (W_e h_{t,s}) for those rows (its own expert, its
// own loads in flight), and the per-row partials meet in LDS, where they are
// summed in slot order. The token-major kernel above runs one wave per row
// tile and loads all slots of a batch in that wave: at a few tokens that is
// half a wave per SIMD. Deterministic: the order of every sum is fixed.
// ---------------------------------------------------------------------------
constexpr int kSplitSlots = 8;

template <int FMT, int LPR, int CPL, int R>
__global__ __launch_bounds__(64 * kSplitSlots) void combine_split_kernel(GatherArgs a) {
    constexpr int RPW = kWave / LPR;
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    constexpr int ROWS = R * RPW;
    constexpr bool AFF = (FMT == INT4AFF);
    constexpr bool KM8 = (FMT == INT8KM);
    static_assert(!KM8 || 32 % ROWS == 0, "int8km: a workgroup's rows within one group");
    constexpr int LUT_HALVES = (FMT == KM4) ? ROWS * 16 : (KM8 ? 256 : 1);   // per wave (slot)
    __shared__ _Float16 lut_lds[kSplitSlots * LUT_HALVES];
    __shared__ float part[kSplitSlots][ROWS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int rsub = lane / LPR;
    const int t = blockIdx.y;
    const int K = a.K;
    const int cpr = (FMT == INT8 || KM8) ? K / 16 : K / 32;
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)code_row_bytes<FMT>(K);
    const int64_t row0 = (int64_t)blockIdx.x * ROWS;
    if (row0 >= a.N) return;   // uniform over the workgroup
    const int last = (int)((a.N - 1 - row0) < ROWS - 1 ? (a.N - 1 - row0) : ROWS - 1);
    // waves past topk repeat the last slot; their partials are not summed
    const int s = wave < a.topk ? wave : a.topk - 1;
    const int e0 = a.ids[t * a.topk + s];
    const int e = e0 < 0 ? 0 : (e0 < a.E ? e0 : a.E - 1);   // clamped, as in the other gather kernels
    const float ws = a.weights[t * a.topk + s];
    const uint8_t *codes_e;
    const void *plane_e;
    expert_slabs<FMT>(a.codes, a.plane, e, a.N, K, codes_e, plane_e);
    uint4 cw[R][CPL];
    float sc[R][CPL];
    float bi[AFF ? R : 1][AFF ? CPL : 1];
#pragma unroll
    for (int g = 0; g < R; g++) {
        int rr = g * RPW + rsub;
        rr = rr <= last ? rr : last;
        const int64_t row = row0 + rr;
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            const int c = sub + LPR * j;
            const int cc = c < cpr ? c : 0;
            cw[g][j] = load_stream16(codes_e + row * (int64_t)row_bytes + (uint32_t)cc * 16u);
            sc[g][j] = plane_scale<FMT>(plane_e, row, nb, cc);
            if constexpr (AFF) bi[g][j] = plane_bias<FMT>(plane_e, row, nb, cc);
        }
    }
    uint32_t xr[CPL][XW];
    float xs[AFF ? CPL : 1];
    const _Float16 *xp = a.x + (int64_t)(a.x_per_slot ? t * a.topk + s : t) * K;
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        const int c = sub + LPR * j;
        load_x_slice<FMT>(xp, c, c < cpr, xr[j]);
        if constexpr (AFF) xs[j] = x_slice_sum<XW>(xr[j]);
    }
    _Float16 *lut_w = lut_lds + wave * LUT_HALVES;
    if constexpr (FMT == KM4) {
        for (int i = lane; i < ROWS * 8; i += kWave) {
            int rr = i / 8;
            rr = rr <= last ? rr : last;
            reinterpret_cast<uint32_t *>(lut_w)[i] = reinterpret_cast<const uint32_t *>(plane_e)[(row0 + rr) * 8 + (i % 8)];
        }
        wave_fence();
    } else if constexpr (KM8) {
#pragma unroll
        for (int q = 0; q < 2; q++)
            reinterpret_cast<uint32_t *>(lut_w)[q * kWave + lane] =
                reinterpret_cast<const uint32_t *>(plane_e)[(row0 / 32) * 128 + q * kWave + lane];
        wave_fence();
    }
    float acc[R];
#pragma unroll
    for (int g = 0; g < R; g++) {
        acc[g] = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            const float d = chunk_dot<FMT>(cw[g][j], xr[j], KM8 ? lut_w : lut_w + (g * RPW + rsub) * 16);
            acc[g] = __builtin_fmaf(d, ws * sc[g][j], acc[g]);
            if constexpr (AFF) acc[g] = __builtin_fmaf(xs[j], ws * bi[g][j], acc[g]);
        }
    }
    using Red = GroupReduce<R, LPR>;
    Red::run(acc, lane);
    if (Red::writer(lane)) {
        const int base = Red::base(lane);
#pragma unroll
        for (int j = 0; j < Red::live; j++) part[wave][(base + j) * RPW + rsub] = acc[j];
    }
    __syncthreads();
    if (threadIdx.x < ROWS && threadIdx.x <= last) {
        float y = 0.f;
        for (int w = 0; w < a.topk; w++) y += part[w][threadIdx.x];   // slot order
        reinterpret_cast<float *>(a.out)[(int64_t)t * a.N + row0 + threadIdx.x] = y;
    }
}

template <int FMT, int LPR, int CPL, int ROWS>
static void launch_combine_split(GatherArgs a, hipStream_t st) {
    constexpr int R = ROWS / (kWave / LPR);
    const int tiles = (int)((a.N + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((combine_split_kernel<FMT, LPR, CPL, R>), dim3(tiles, a.T), dim3(64 * kSplitSlots), 0, st, a);
}

template <int FMT, int LPR, int CPL>
static hipError_t launch_token_major(GatherArgs a, hipStream_t st) {
    if (CPL == 1 && a.topk <= kSplitSlots) {   // longer rows keep the token-major kernel (registers)
        // measured on MI355X, int4 down 2048 x 512, top-8 of 256, HIP graphs:
        // T = 1 3.5 us (8 rows per workgroup) against 5.0 for the token-major
        // kernel, T = 4 5.8 (16 rows) against 8.4, T = 8 8.4 (16 rows) against 12.8
        constexpr int ROWS_FEW = (LPR == 64) ? 4 : 8, ROWS_MANY = (LPR == 64) ? 4 : 16;
        if (a.T <= 2) launch_combine_split<FMT, LPR, CPL, ROWS_FEW>(a, st);
        else launch_combine_split<FMT, LPR, CPL, ROWS_MANY>(a, st);
        return hipGetLastError();
    }
    constexpr int R = (LPR == 64) ? 4 : 1;
    constexpr int ROWS = R * (kWave / LPR);
    // few tokens: few waves, so each takes as many slots per round trip as
    // registers allow; more tokens: smaller batches keep more waves resident
    constexpr int SB_WIDE = combine_slot_batch<FMT, R, CPL>();
    constexpr int SB_NARROW = SB_WIDE < 4 ? SB_WIDE : 4;
    int tiles = (int)((a.N + ROWS - 1) / ROWS);
    if (a.T <= 4)
        hipLaunchKernelGGL((combine_gather_kernel<FMT, LPR, CPL, R, SB_WIDE>), dim3(tiles, a.T), dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((combine_gather_kernel<FMT, LPR, CPL, R, SB_NARROW>), dim3(tiles, a.T), dim3(64), 0, st,
                           a);
    return hipGetLastError();
}

// dispatch on the row length: lanes per row and chunks per lane
template <int FMT, int EPI, bool FUSED>
static hipError_t launch_shape(GatherArgs a, int umax, bool *handled, hipStream_t st) {
    constexpr int E = ChunkTraits<FMT>::kElems;
    const int cpr = a.K / E;
    *handled = true;
    if constexpr (EPI == EPI_COMBINE) {
        (void)umax;
        if (cpr <= 16) return launch_token_major<FMT, 16, 1>(a, st);
        if (cpr <= 32) return launch_token_major<FMT, 32, 1>(a, st);
        if (cpr <= 64) return launch_token_major<FMT, 64, 1>(a, st);
        if (cpr <= 128) return launch_token_major<FMT, 64, 2>(a, st);
        if (cpr <= 192) return launch_token_major<FMT, 64, 3>(a, st);
        if (cpr <= 256) return launch_token_major<FMT, 64, 4>(a, st);
    } else {
        if (cpr <= 16) return launch_expert_major<FMT, 16, 1, EPI, FUSED>(a, umax, st);
        if (cpr <= 32) return launch_expert_major<FMT, 32, 1, EPI, FUSED>(a, umax, st);
        if (cpr <= 64) return launch_expert_major<FMT, 64, 1, EPI, FUSED>(a, umax, st);
        if (cpr <= 128) return launch_expert_major<FMT, 64, 2, EPI, FUSED>(a, umax, st);
        if (cpr <= 192) return launch_expert_major<FMT, 64, 3, EPI, FUSED>(a, umax, st);
        if (cpr <= 256) return launch_expert_major<FMT, 64, 4, EPI, FUSED>(a, umax, st);
    }
    *handled = false;
    return hipSuccess;
}

template <int FMT>
static hipError_t launch_fmt(GatherArgs a, int epi, bool fused, int umax, bool *handled, hipStream_t st) {
    if (epi == EPI_COMBINE) return launch_shape<FMT, EPI_COMBINE, false>(a, umax, handled, st);
    if (epi == EPI_SWIGLU)
        return fused ? launch_shape<FMT, EPI_SWIGLU, true>(a, umax, handled, st)
                     : launch_shape<FMT, EPI_SWIGLU, false>(a, umax, handled, st);
    return launch_shape<FMT, EPI_NONE, false>(a, umax, handled, st);
}

static hipError_t launch_any(int fmt, GatherArgs a, int epi, bool fused, int umax, hipStream_t st) {
    bool handled = false;
    hipError_t err;
    switch (fmt) {
    case INT4: err = launch_fmt<INT4>(a, epi, fused, umax, &handled, st); break;
    case FP4: err = launch_fmt<FP4>(a, epi, fused, umax, &handled, st); break;
    case INT8: err = launch_fmt<INT8>(a, epi, fused, umax, &handled, st); break;
    case KM4: err = launch_fmt<KM4>(a, epi, fused, umax, &handled, st); break;
    case INT8KM: err = launch_fmt<INT8KM>(a, epi, fused, umax, &handled, st); break;
    default: err = launch_fmt<INT4AFF>(a, epi, fused, umax, &handled, st); break;
    }
    if (err != hipSuccess) return err;
    return handled ? hipSuccess : hipErrorInvalidValue;
}

static GatherArgs make_args(const void *codes, const void *plane, int E, int64_t N, int64_t K, const void *x,
                            int x_per_slot, int T, int topk, const int32_t *ids, const float *weights, void *out) {
    GatherArgs a;
    a.codes = reinterpret_cast<const uint8_t *>(codes);
    a.plane = plane;
    a.E = E;
    a.N = N;
    a.K = (int)K;
    a.x = reinterpret_cast<const _Float16 *>(x);
    a.x_per_slot = x_per_slot;
    a.T = T;
    a.topk = topk;
    a.ids = ids;
    a.weights = weights;
    a.logits = nullptr;
    a.ids_out = nullptr;
    a.weights_out = nullptr;
    a.out = out;
    a.out_rows = N;
    a.tile_rows = 0;
    return a;
}

hipError_t launch_gather(int fmt, const void *codes, const void *plane, int E, int64_t N, int64_t K, const void *x,
                         qmv_dtype xdt, int x_per_slot, int T, int topk, const int32_t *ids, const float *weights,
                         int epi, void *y, void *workspace, hipStream_t st) {
    (void)xdt;
    (void)workspace;
    GatherArgs a = make_args(codes, plane, E, N, K, x, x_per_slot, T, topk, ids, weights, y);
    if (epi == EPI_SWIGLU) a.out_rows = N / 2;
    int umax = T * topk < E ? T * topk : E;
    return launch_any(fmt, a, epi, false, umax, st);
}

hipError_t launch_moe_ffn(int fmt, const void *gu_codes, const void *gu_plane, const void *dn_codes,
                          const void *dn_plane, int E, int64_t H, int64_t I, const float *logits, const void *x, int T,
                          int topk, int32_t *ids, float *weights, void *h, float *y, hipStream_t st) {
    // gate/up + SwiGLU (h [T][topk][I]). For one token the routing is fused
    // into it: each workgroup routes the token itself, which costs less than
    // a separate launch. Beyond one token the duplicated routing work grows
    // with T times the number of workgroups and a separate routing launch is
    // cheaper.
    GatherArgs g = make_args(gu_codes, gu_plane, E, 2 * I, H, x, 0, T, topk, ids, weights, h);
    g.out_rows = I;
    const bool fuse = (T == 1);
    if (fuse) {
        g.logits = logits;
        g.ids_out = ids;
        g.weights_out = weights;
    } else {
        hipError_t err = launch_moe_route(logits, T, E, topk, ids, weights, st);
        if (err != hipSuccess) return err;
    }
    int umax = T * topk < E ? T * topk : E;
    hipError_t err = launch_any(fmt, g, EPI_SWIGLU, fuse, umax, st);
    if (err != hipSuccess) return err;
    // launch 2: down projection with the weighted combine (y [T][H])
    GatherArgs d = make_args(dn_codes, dn_plane, E, H, I, h, 1, T, topk, ids, weights, y);
    return launch_any(fmt, d, EPI_COMBINE, false, umax, st);
}

}  // namespace qmv
