// emu_kernels.hip -- the split combination kernel and the dispatch of the
// main kernel's variants (emu_main_kernel.h, instantiated by emu_variant.hip).
#include <hip/hip_runtime.h>

#include "emu_internal.h"
#include "emu_output.h"
#include "fp_round.h"

namespace emu {

namespace {

// Combination of the split partials, then the epilogue; binary32 adds in
// the default round-to-nearest-even mode.  Serial: ((p0 + p1) + p2) + ...
// Pairwise: the stride-halving tree over P = the next power of two >= S
// (for h = P/2 .. 1: p_i += p_{i+h} where i + h < S; S = 3 gives
// (p0 + p2) + p1), run as that loop: in registers for S <= 16, in the
// workspace beyond (no indexed local arrays, so no scratch memory).  CHUNKED: the
// partials are slow-mode chunk results, cps per split (a separate kernel, so
// that the one-partial-per-split case keeps its own simpler code).
template <bool CHUNKED>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.M * p.N;
    if (idx >= total) return;
    const int64_t m = idx / p.N, n = idx - m * p.N;
    // split s's partial: its single partial, or the running binary32 sum of
    // its slow-mode chunk results in order from +0 (chunk results are never
    // -0, so the first add reproduces the first chunk bit for bit).  Eight
    // loads are issued before their adds, which stay in order.
    constexpr int U = 8;
    auto ordered_sum = [&](const float *q, int n, int64_t stride, float a) {
        int c = 0;
        for (; c + U <= n; c += U) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = q[(int64_t)(c + u) * stride];
#pragma unroll
            for (int u = 0; u < U; ++u) a = a + v[u];
        }
        for (; c < n; ++c) a = a + q[(int64_t)c * stride];
        return a;
    };
    auto split_partial = [&](int s) {
        const float *q = p.part + (int64_t)s * p.cps * total + idx;
        if (!CHUNKED) return q[0];
        return ordered_sum(q, p.cps, total, 0.0f);
    };
    float acc;
    if (!p.pairwise) {
        acc = split_partial(0);
        for (int s = 1; s < p.S; ++s) acc = acc + split_partial(s);
    } else if (p.S <= 16) {
        // The stride-halving tree itself, over 16 slots with fixed indices
        // (registers): strides of S or more add nothing, so it is the tree
        // over P for every S <= 16, each addition in the same order.
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = i < p.S ? split_partial(i) : 0.0f;
#pragma unroll
        for (int h = 8; h >= 1; h >>= 1)
#pragma unroll
            for (int i = 0; i < h; ++i)
                if (i + h < p.S) v[i] = v[i] + v[i + h];
        acc = v[0];
    } else {
        // More splits: the same loop in place over this output's column of
        // the workspace, each split's partial in its first slot (a stored
        // chunk sum overwrites the split's first chunk after all of its
        // chunks are read); every slot is read and written by this thread only.
        float *q = p.part + idx;
        const int64_t ss = (int64_t)p.cps * total;
        if (CHUNKED)
            for (int s = 0; s < p.S; ++s) q[s * ss] = split_partial(s);
        int P = 1;
        while (P < p.S) P <<= 1;
        for (int h = P >> 1; h >= 1; h >>= 1)
            for (int i = 0; i + h < p.S && i < h; ++i) q[i * ss] = q[i * ss] + q[(i + h) * ss];
        acc = q[0];
    }
    uint32_t alpha = 0, sr = 0x3F800000u;
    if (p.out_kind != OUT_ACC_F32) {
        alpha = mul_f32(__float_as_uint(*p.scale_x), __float_as_uint(*p.scale_w));
        sr = scale_result_bits(p.scale_result);
    }
    store_epilogue(p.out_kind, p.out, m * p.ldo + n, __float_as_uint(acc), alpha, sr);
}

}  // namespace

TileShape tile_shape(int cfg)
{
    switch (cfg) {
    case TILE_64x128: return {64, 128, 256};
    case TILE_64x64: return {64, 64, 256};
    case TILE_32x64: return {32, 64, 256};
    case TILE_32x32: return {32, 32, 256};
    case TILE_16x16_G2: return {16, 16, 512};
    case TILE_16x16_G4: return {16, 16, 1024};
    case TILE_64x64_MX: return {64, 64, 256};
    case TILE_64x128_MX: return {64, 128, 256};
    case TILE_16x8_G4: return {16, 8, 512};
    case TILE_16x64_MX: return {16, 64, 64};
    case TILE_32x32_S4: return {32, 32, 256};
    case TILE_32x32_MX_S4: return {32, 32, 256};
    case TILE_32x16_MX_S5: return {32, 16, 256};
    default: return {64, 128, 256};
    }
}

hipError_t launch_main(int cfg, int block, int xfmt, int wfmt, const MainParams &p, int S, hipStream_t stream)
{
    const int key = (block << 4) | (xfmt << 1) | wfmt;
    switch (key) {
    case (32 << 4) | 0: return launch_variant<32, 0, 0>(cfg, p, S, stream);
    case (32 << 4) | 1: return launch_variant<32, 0, 1>(cfg, p, S, stream);
    case (32 << 4) | 2: return launch_variant<32, 1, 0>(cfg, p, S, stream);
    case (16 << 4) | 0: return launch_variant<16, 0, 0>(cfg, p, S, stream);
    case (16 << 4) | 1: return launch_variant<16, 0, 1>(cfg, p, S, stream);
    case (16 << 4) | 2: return launch_variant<16, 1, 0>(cfg, p, S, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_main_cin(int cfg, int block, int xfmt, int wfmt, const MainParams &p, hipStream_t stream)
{
    const int key = (block << 4) | (xfmt << 1) | wfmt;
    switch (key) {
    case (32 << 4) | 0: return launch_variant_cin<32, 0, 0>(cfg, p, stream);
    case (32 << 4) | 1: return launch_variant_cin<32, 0, 1>(cfg, p, stream);
    case (32 << 4) | 2: return launch_variant_cin<32, 1, 0>(cfg, p, stream);
    case (16 << 4) | 0: return launch_variant_cin<16, 0, 0>(cfg, p, stream);
    case (16 << 4) | 1: return launch_variant_cin<16, 0, 1>(cfg, p, stream);
    case (16 << 4) | 2: return launch_variant_cin<16, 1, 0>(cfg, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine(const CombineParams &p, hipStream_t stream)
{
    const int64_t total = (int64_t)p.M * p.N;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (p.cps > 1)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace emu
