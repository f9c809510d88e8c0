// Mixture-of-experts decode: top-k routing and the routed-expert gather
// matvec ("Stream D - Quantization (FP4 + QAT-int4)...", section 1: the
// gather_qmm kernels over expert slabs blocked along K; "Dense-path int4km
// coverage + flagship Qwen3.6-35B...", section 1: only the routed experts'
// weights are read, avoiding the all-experts over-read).
//
// gfx950 design. Decode moves at most T*topk experts; each workgroup works
// on one (unique expert, row tile) pair. The expert list is rebuilt in every
// workgroup from the T*topk ids (at most 64 entries, a few hundred cycles),
// so there is no separate bucketing launch and no host synchronization. The
// tokens that chose an expert are processed against the same weight tile,
// so a chosen expert's bytes come from HBM once; a second pair of tokens
// re-reads the tile from L2. SwiGLU is fused into the gate/up pass; the
// down pass writes one fp32 row per (token, slot) and a small combine
// kernel sums the slots in slot order, so results are deterministic.
#include "qmv_device.h"
#include "qmv_launch.h"

namespace qmv {

// ---------------------------------------------------------------------------
// routing: one wave per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int T, int E, int topk,
                                                    int32_t *__restrict__ ids, float *__restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *l = logits + (int64_t)t * E;
    uint64_t taken = 0;
    float my_v = 0.f;
    int my_i = 0;
    for (int j = 0; j < topk; j++) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
        for (int i = 0; lane + 64 * i < E; i++) {
            int e = lane + 64 * i;
            if (taken & (1ull << i)) continue;
            float v = l[e];
            if (v > bv || (v == bv && e < bi)) {
                bv = v;
                bi = e;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            float ov = __shfl_xor(bv, m);
            int oi = __shfl_xor(bi, m);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
        if (lane == j) {
            my_v = bv;
            my_i = bi;
        }
    }
    const float vmax = __shfl(my_v, 0);
    float p = lane < topk ? expf(my_v - vmax) : 0.f;
    float z = p;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m);
    if (lane < topk) {
        ids[(int64_t)t * topk + lane] = my_i;
        weights[(int64_t)t * topk + lane] = p / z;
    }
}

hipError_t launch_moe_route(const float *logits, int T, int E, int topk, int32_t *ids, float *weights,
                            hipStream_t st) {
    hipLaunchKernelGGL(route_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, topk, ids, weights);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gather matvec
// ---------------------------------------------------------------------------
enum Epi { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_COMBINE = 2 };

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
    void *out;          // NONE/COMBINE: fp32 rows per pair; SWIGLU: fp16 rows per pair
    int64_t out_rows;   // logical rows per pair (N, or N/2 for SWIGLU)
    int tile_rows;      // logical rows per workgroup
};

template <int FMT>
__device__ __forceinline__ float plane_scale(const void *plane, int64_t row, int nb, int c) {
    if constexpr (FMT == INT4 || FMT == INT8) {
        int blk = (FMT == INT8) ? c / 2 : c;
        return f16_bits_to_f32(reinterpret_cast<const uint16_t *>(plane)[row * nb + blk]);
    } else if constexpr (FMT == FP4) {
        return e8m0_to_f32(reinterpret_cast<const uint8_t *>(plane)[row * nb + c]);
    } else {
        return 1.f;
    }
}

// One pass over the workgroup's row tile for PB token slots (pairs).
// R row groups per wave iteration; with SWIGLU the first R/2 groups are gate
// rows and the last R/2 the matching up rows.
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
    const int cpr = (FMT == INT8) ? K / 16 : K / 32;
    const int nb = K / 32;
    const int64_t row_bytes = (FMT == INT8) ? K : K / 2;

    uint32_t xr[CPL][PB][XW];
#pragma unroll
    for (int p = 0; p < PB; p++) {
        int pr = pairs[p];
        const _Float16 *xp = a.x + (int64_t)(a.x_per_slot ? pr : pr / a.topk) * K;
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            int c = sub + LPR * j;
            load_x_slice<FMT>(xp, c, c < cpr, xr[j][p]);
        }
    }
    const int64_t tile0 = (int64_t)blockIdx.x * a.tile_rows;
    int64_t tile1 = tile0 + a.tile_rows;
    if (tile1 > a.out_rows) tile1 = a.out_rows;
    for (int64_t l0 = tile0 + (int64_t)wave * LROWS; l0 < tile1; l0 += 4 * LROWS) {
        uint4 cw[R][CPL];
        float sc[R][CPL];
        int64_t prow[R];
        bool rvalid[R];
#pragma unroll
        for (int g = 0; g < R; g++) {
            int gl = (EPI == EPI_SWIGLU) ? (g % G) : g;
            int64_t lrow = l0 + gl * RPW + rsub;
            rvalid[g] = lrow < tile1;
            prow[g] = (EPI == EPI_SWIGLU && g >= G) ? lrow + a.out_rows : lrow;
            const uint8_t *rp = codes_e + (rvalid[g] ? prow[g] : 0) * row_bytes;
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                int c = sub + LPR * j;
                bool v = rvalid[g] && c < cpr;
                cw[g][j] = v ? *reinterpret_cast<const uint4 *>(rp + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
                sc[g][j] = v ? plane_scale<FMT>(plane_e, prow[g], nb, c) : 0.f;
            }
        }
        if constexpr (FMT == KM4) {
            const uint32_t *lsrc = reinterpret_cast<const uint32_t *>(plane_e);
            uint32_t *ldst = reinterpret_cast<uint32_t *>(lut_w);
            for (int i = lane; i < R * RPW * 8; i += kWave) {
                int g = i / (RPW * 8), rs = (i / 8) % RPW;
                int gl = (EPI == EPI_SWIGLU) ? (g % G) : g;
                int64_t lrow = l0 + gl * RPW + rs;
                int64_t pr = (EPI == EPI_SWIGLU && g >= G) ? lrow + a.out_rows : lrow;
                ldst[i] = lrow < tile1 ? lsrc[pr * 8 + (i % 8)] : 0u;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        float acc[R][PB];
#pragma unroll
        for (int g = 0; g < R; g++)
#pragma unroll
            for (int p = 0; p < PB; p++) acc[g][p] = 0.f;
#pragma unroll
        for (int g = 0; g < R; g++)
#pragma unroll
            for (int j = 0; j < CPL; j++)
#pragma unroll
                for (int p = 0; p < PB; p++) {
                    float d;
                    if constexpr (FMT == INT4) d = chunk_dot_int4(cw[g][j], xr[j][p]);
                    else if constexpr (FMT == FP4) d = chunk_dot_fp4(cw[g][j], xr[j][p]);
                    else if constexpr (FMT == INT8) d = chunk_dot_int8(cw[g][j], xr[j][p]);
                    else d = chunk_dot_km4(cw[g][j], lut_w + (g * RPW + rsub) * 16, xr[j][p]);
                    acc[g][p] = __builtin_fmaf(d, sc[g][j], acc[g][p]);
                }
        if constexpr (FMT == KM4) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
#pragma unroll
        for (int g = 0; g < R; g++)
#pragma unroll
            for (int p = 0; p < PB; p++) acc[g][p] = group_sum<LPR>(acc[g][p]);
        if (sub == 0) {
#pragma unroll
            for (int g = 0; g < G; g++) {
                int64_t lrow = l0 + g * RPW + rsub;
                if (lrow >= tile1) continue;
#pragma unroll
                for (int p = 0; p < PB; p++) {
                    int64_t o = (int64_t)pairs[p] * a.out_rows + lrow;
                    if constexpr (EPI == EPI_SWIGLU) {
                        float gt = acc[g][p], up = acc[g + G][p];
                        float h = gt / (1.0f + expf(-gt)) * up;
                        reinterpret_cast<_Float16 *>(a.out)[o] = (_Float16)h;
                    } else {
                        reinterpret_cast<float *>(a.out)[o] = acc[g][p];
                    }
                }
            }
        }
    }
}

template <int FMT, int LPR, int CPL, int R, int EPI>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    constexpr int RPW = kWave / LPR;
    __shared__ int s_ids[512];
    __shared__ uint32_t s_bits[128];   // one bit per expert id (E <= 4096)
    __shared__ int s_pairs[8];
    __shared__ int s_np;
    __shared__ int s_expert;
    __shared__ _Float16 lut_lds[(FMT == KM4) ? 4 * R * RPW * 16 : 1];
    const int tid = threadIdx.x;
    const int npairs = a.T * a.topk;
    const int u = blockIdx.y;
    for (int i = tid; i < 128; i += blockDim.x) s_bits[i] = 0;
    __syncthreads();
    for (int i = tid; i < npairs; i += blockDim.x) {
        int e = a.ids[i];
        s_ids[i] = e;
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
        int np = 0;
        for (int i = 0; i < npairs && found >= 0; i++)
            if (s_ids[i] == found && np < 8) s_pairs[np++] = i;
        s_np = np;
    }
    __syncthreads();
    const int e = s_expert;
    if (e < 0) return;
    const int np = s_np;
    const int64_t row_bytes = (FMT == INT8) ? a.K : a.K / 2;
    const uint8_t *codes_e = a.codes + (int64_t)e * a.N * row_bytes;
    const void *plane_e;
    if constexpr (FMT == FP4)
        plane_e = reinterpret_cast<const uint8_t *>(a.plane) + (int64_t)e * a.N * (a.K / 32);
    else if constexpr (FMT == KM4)
        plane_e = reinterpret_cast<const uint16_t *>(a.plane) + (int64_t)e * a.N * 16;
    else
        plane_e = reinterpret_cast<const uint16_t *>(a.plane) + (int64_t)e * a.N * (a.K / 32);
    _Float16 *lut_w = lut_lds + (tid >> 6) * R * RPW * 16;
    int p0 = 0;
    for (; p0 + 2 <= np; p0 += 2)
        gather_pass<FMT, 2, LPR, CPL, R, EPI>(a, codes_e, plane_e, s_pairs + p0, lut_w);
    if (p0 < np) gather_pass<FMT, 1, LPR, CPL, R, EPI>(a, codes_e, plane_e, s_pairs + p0, lut_w);
}

// y[t][n] = sum over slots (in order) of weights[t][slot] * part[t*topk+slot][n]
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ part, const float *__restrict__ w,
                                                      int T, int topk, int64_t N, float *__restrict__ y) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)T * N) return;
    int t = (int)(gid / N);
    int64_t n = gid % N;
    float acc = 0.f;
    for (int s = 0; s < topk; s++) acc = __builtin_fmaf(w[t * topk + s], part[((int64_t)t * topk + s) * N + n], acc);
    y[gid] = acc;
}

size_t gather_workspace_bytes(int T, int topk, int E, int64_t N, int epi) {
    (void)E;
    if (epi != EPI_COMBINE) return 0;
    return (size_t)T * topk * N * sizeof(float);
}

template <int FMT, int LPR, int CPL, int EPI>
static hipError_t launch_gather_t(GatherArgs a, int umax, hipStream_t st) {
    constexpr int R = (EPI == EPI_SWIGLU) ? 4 : 2;
    constexpr int RPW = kWave / LPR;
    constexpr int G = (EPI == EPI_SWIGLU) ? R / 2 : R;
    // each wave takes two iterations of its tile
    a.tile_rows = 4 * G * RPW * 2;
    int tiles = (int)((a.out_rows + a.tile_rows - 1) / a.tile_rows);
    hipLaunchKernelGGL((gather_kernel<FMT, LPR, CPL, R, EPI>), dim3(tiles, umax), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int FMT, int EPI>
static hipError_t launch_gather_shape(GatherArgs a, int umax, bool *handled, hipStream_t st) {
    constexpr int E = ChunkTraits<FMT>::kElems;
    const int cpr = a.K / E;
    *handled = true;
    if (cpr <= 16) return launch_gather_t<FMT, 16, 1, EPI>(a, umax, st);
    if (cpr <= 32) return launch_gather_t<FMT, 32, 1, EPI>(a, umax, st);
    if (cpr <= 64) return launch_gather_t<FMT, 64, 1, EPI>(a, umax, st);
    if (cpr <= 128) return launch_gather_t<FMT, 64, 2, EPI>(a, umax, st);
    if (cpr <= 192) return launch_gather_t<FMT, 64, 3, EPI>(a, umax, st);
    if (cpr <= 256) return launch_gather_t<FMT, 64, 4, EPI>(a, umax, st);
    *handled = false;
    return hipSuccess;
}

template <int FMT>
static hipError_t launch_gather_fmt(GatherArgs a, int epi, int umax, bool *handled, hipStream_t st) {
    if (epi == EPI_SWIGLU) return launch_gather_shape<FMT, EPI_SWIGLU>(a, umax, handled, st);
    return launch_gather_shape<FMT, EPI_NONE>(a, umax, handled, st);
}

hipError_t launch_gather(int fmt, const void *codes, const void *plane, int E, int64_t N, int64_t K, const void *x,
                         qmv_dtype xdt, int x_per_slot, int T, int topk, const int32_t *ids, const float *weights,
                         int epi, void *y, void *workspace, hipStream_t st) {
    (void)xdt;
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
    a.out = (epi == EPI_COMBINE) ? workspace : y;
    a.out_rows = (epi == EPI_SWIGLU) ? N / 2 : N;
    a.tile_rows = 0;
    int umax = T * topk < E ? T * topk : E;
    bool handled = false;
    hipError_t err;
    switch (fmt) {
    case INT4: err = launch_gather_fmt<INT4>(a, epi, umax, &handled, st); break;
    case FP4: err = launch_gather_fmt<FP4>(a, epi, umax, &handled, st); break;
    case INT8: err = launch_gather_fmt<INT8>(a, epi, umax, &handled, st); break;
    default: err = launch_gather_fmt<KM4>(a, epi, umax, &handled, st); break;
    }
    if (err != hipSuccess) return err;
    if (!handled) return hipErrorInvalidValue;
    if (epi == EPI_COMBINE) {
        int64_t tot = (int64_t)T * N;
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                           reinterpret_cast<const float *>(workspace), weights, T, topk, N,
                           reinterpret_cast<float *>(y));
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace qmv
