// Register-only MFMA rate probe for gfx950: a measurement aid that bounds
// what any bf16 v_mfma_f32_32x32x16_bf16 kernel can sustain on this chip,
// not a step of the indexer or the attention.
//
// Every wave runs four independent accumulation chains of 32x32x16 bf16
// MFMAs whose operands never leave registers: no LDS, no memory traffic
// except one float per lane stored at the end.  The operands are
// pseudo-random bf16 values drawn per lane from a xorshift generator; with
// `rotate` set, consecutive MFMAs cycle through four different operand
// fragments per side so that the matrix inputs change on every issue, as
// they do in a real contraction.  The achieved rate against the nominal
// peak shows how far the clock drops under the matrix pipe's own power
// draw with realistic operand bits.
#include "csa_indexer.h"
#include "csa_internal.h"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

template <bool ROTATE>
__global__ __launch_bounds__(256) void probe_mfma_kernel(float *out, int iters)
{
    bf16x8 av[4], bv[4];
    uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            h ^= h << 13; h ^= h >> 17; h ^= h << 5;
            av[f][i] = (__bf16)(((float)(h & 0xFFFF) - 32768.0f) * 1e-5f);
            h ^= h << 13; h ^= h >> 17; h ^= h << 5;
            bv[f][i] = (__bf16)(((float)(h & 0xFFFF) - 32768.0f) * 1e-5f);
        }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ROTATE ? (u + c) & 3 : 0],
                                                                 bv[ROTATE ? (u + 3 * c) & 3 : 0], acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace csa

extern "C" int csa_probe_mfma(float *out, int32_t blocks, int32_t iters, int32_t rotate, void *stream_ptr)
{
    hipStream_t stream = (hipStream_t)stream_ptr;
    if (out == nullptr) return CSA_ERR_NULL_PTR;
    if (blocks < 1 || blocks > (1 << 20) || iters < 4 || iters > (1 << 24) || iters % 4 != 0)
        return CSA_ERR_BAD_SHAPE;
    if (((uintptr_t)out & 3) != 0) return CSA_ERR_MISALIGNED;
    if (rotate) csa::probe_mfma_kernel<true><<<dim3((unsigned)blocks), 256, 0, stream>>>(out, iters);
    else csa::probe_mfma_kernel<false><<<dim3((unsigned)blocks), 256, 0, stream>>>(out, iters);
    return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}
