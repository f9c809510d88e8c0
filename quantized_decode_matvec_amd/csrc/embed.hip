// Embedding dequant-gather for an int8 table with one fp16 scale per row:
// out[t][h] = fp16(q[ids[t]][h] * scale[ids[t]]) ("coreai-optimization
// reference", "The LM head + embeddings": the front-end table gather is a
// plain int8 per-row dequant-gather, kept out of the decode core).
//
// gfx950 design: the gather is a pure copy-and-convert, bound by the bytes of
// the chosen rows (H int8 in, 2H out per token). A thread converts 8 values:
// one 8-byte load, one scale, eight exact fp32 products rounded once to
// fp16, one 16-byte store. Ids outside [0, V) produce a zero row instead of
// reading outside the table.
#include "qmv_device.h"
#include "qmv_launch.h"

namespace qmv {

__global__ __launch_bounds__(256) void embed_gather_int8_kernel(const int8_t *__restrict__ codes,
                                                                const uint16_t *__restrict__ scale, int64_t V,
                                                                int64_t H, const int32_t *__restrict__ ids,
                                                                _Float16 *__restrict__ out) {
    const int64_t t = blockIdx.y;
    const int64_t h0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (h0 >= H) return;
    const int32_t v = ids[t];
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (v >= 0 && v < V) {
        const float s = f16_bits_to_f32(scale[v]);
        const uint2 q = *reinterpret_cast<const uint2 *>(codes + (int64_t)v * H + h0);
        uint32_t r[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t word = i < 2 ? q.x : q.y;
            const int sh = 16 * (i & 1);
            const float a = (float)(int8_t)(word >> sh), b = (float)(int8_t)(word >> (sh + 8));
            h2 p;
            p.x = (_Float16)(a * s);   // exact product, one rounding (nearest even)
            p.y = (_Float16)(b * s);
            r[i] = as_u32(p);
        }
        o = make_uint4(r[0], r[1], r[2], r[3]);
    }
    *reinterpret_cast<uint4 *>(out + t * H + h0) = o;
}

hipError_t launch_embed_gather_int8(const int8_t *codes, const uint16_t *scale, int64_t V, int64_t H,
                                    const int32_t *ids, int64_t T, void *out, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int64_t per_block = 256 * 8;
    dim3 grid((unsigned)((H + per_block - 1) / per_block), (unsigned)T);
    hipLaunchKernelGGL(embed_gather_int8_kernel, grid, dim3(256), 0, st, codes, scale, V, H, ids,
                       reinterpret_cast<_Float16 *>(out));
    return hipGetLastError();
}

}  // namespace qmv
