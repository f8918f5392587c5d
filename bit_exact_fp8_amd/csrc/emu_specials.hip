// emu_specials.hip -- infinities resolved after the main kernel, for large
// problems: a pass over the e5m2 operand's rows that lists where their
// infinities are, and a fix-up of the outputs those rows touch.
//
// The rule (validation page, claims table: NaN and Inf rows and columns
// through the GEMM epilogue; IEEE products and sums): an output whose two
// rows pair an infinity with a zero, or give infinite products of both
// signs, is NaN; otherwise it is the infinity of its infinite products'
// sign.  It depends only on the k where a row holds an infinity, so the
// work per output is the number of infinities in its rows, not K.  NaN
// codes are left to the main kernel: its row flags give those outputs the
// canonical NaN directly.
#include <hip/hip_runtime.h>

#include "emu_main_kernel.h"
#include "emu_output.h"

namespace emu {

namespace {

constexpr int kRowWaves = 4;  // A rows per row-kernel workgroup, one per wave

// One wave per A row: 16 codes per lane and load, 1 KiB per wave.
__global__ __launch_bounds__(256) void inf_rows_kernel(DeferParams p)
{
    __shared__ uint32_t cnt[kRowWaves], nanf[kRowWaves];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowWaves + wv;
    if (lane == 0) {
        cnt[wv] = 0u;
        nanf[wv] = 0u;
    }
    __syncthreads();
    if (row < p.ra) {
        const uint8_t *r = p.a + row * p.lda;
        uint32_t nan = 0;
        for (int64_t k = (int64_t)lane * 16; k < p.K; k += 1024) {
            const uint4 v = *reinterpret_cast<const uint4 *>(r + k);
            const uint32_t vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                nan |= nan_bytes<FMT_E5M2>(vs[u]);
                uint32_t m = inf_bytes<FMT_E5M2>(vs[u]);
                while (m) {  // rare: one list slot per infinity
                    const int byte = __builtin_ctz(m) >> 3;
                    const uint32_t slot = atomicAdd(&cnt[wv], 1u);
                    if (slot < (uint32_t)kDeferCap)
                        p.pos[row * kDeferCap + slot] =
                            (uint32_t)(k + 4 * u + byte) | (((vs[u] >> (8 * byte + 7)) & 1u) << 31);
                    m &= m - 1u;
                }
            }
        }
        if (nan) atomicOr(&nanf[wv], 1u);
    }
    __syncthreads();
    if (row < p.ra && lane == 0) p.info[row] = nanf[wv] ? 0u : cnt[wv];
}

// Workgroup (x, y): B rows [x * b_rows, ...) staged in LDS, A rows
// [y * a_rows, ...).  Workgroups whose A rows hold no listed infinity leave
// at once; the others stage their B rows (noting those that hold a NaN
// code) and resolve every (A row, B row) pair with info != 0.  Consecutive
// lanes take consecutive output columns where the layout allows.
__global__ __launch_bounds__(256) void inf_fixup_kernel(DeferParams p)
{
    extern __shared__ uint4 lds4[];
    __shared__ uint32_t bnan[16];
    const int t = threadIdx.x;
    const int64_t a0 = (int64_t)blockIdx.y * p.a_rows;
    const int na = (int)((p.ra - a0 < p.a_rows) ? p.ra - a0 : p.a_rows);
    uint32_t any = 0;
    for (int i = t; i < na; i += 256) any |= p.info[a0 + i];
    if (!__syncthreads_or(any != 0u)) return;

    const int64_t b0 = (int64_t)blockIdx.x * p.b_rows;
    const int nb = (int)((p.rb - b0 < p.b_rows) ? p.rb - b0 : p.b_rows);
    const int64_t Kp = p.K + 16;
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds4);
    if (t < 16) bnan[t] = (t < nb) ? 0u : 1u;
    __syncthreads();
    const int64_t q16 = p.K >> 4;
    for (int r = 0; r < nb; ++r) {
        const uint8_t *src = p.b + (b0 + r) * p.ldb;
        uint32_t nan = 0;
        for (int64_t q = t; q < q16; q += 256) {
            const uint4 v = *reinterpret_cast<const uint4 *>(src + q * 16);
            *reinterpret_cast<uint4 *>(lds + r * Kp + q * 16) = v;
            nan |= has_special<FMT_E4M3>(v.x) | has_special<FMT_E4M3>(v.y) | has_special<FMT_E4M3>(v.z) |
                   has_special<FMT_E4M3>(v.w);  // e4m3fn: NaN is its only special code
        }
        if (nan) atomicOr(&bnan[r], 1u);
    }
    __syncthreads();

    uint32_t alpha = 0, sr = 0x3F800000u;
    if (p.out_kind != OUT_ACC_F32) {
        alpha = mul_f32(__float_as_uint(*p.scale_x), __float_as_uint(*p.scale_w));
        sr = scale_result_bits(p.scale_result);
    }
    const int npairs = na * p.b_rows;
    for (int idx = t; idx < npairs; idx += 256) {
        int al, r;
        if (p.a_is_w) {
            al = idx % na;
            r = idx / na;
        } else {
            r = idx % p.b_rows;
            al = idx / p.b_rows;
        }
        const int64_t a = a0 + al;
        const uint32_t cnt = p.info[a];
        if (!cnt || bnan[r]) continue;
        const uint8_t *br = lds + r * Kp;
        uint32_t bad = 0, pos = 0, neg = 0;
        if (cnt <= (uint32_t)kDeferCap) {
            const uint32_t *e = p.pos + a * kDeferCap;
            for (uint32_t i = 0; i < cnt; ++i) {
                const uint32_t v = e[i];
                const uint32_t bc = br[v & 0x7FFFFFFFu];
                bad |= ((bc & 0x7Fu) == 0u) ? 1u : 0u;  // infinity times zero
                const uint32_t s = (v >> 31) ^ (bc >> 7);
                neg |= s;
                pos |= s ^ 1u;
            }
        } else {  // more infinities than the list holds: the whole A row
            const uint8_t *ar = p.a + a * p.lda;
            for (int64_t k = 0; k < p.K; k += 16) {
                const uint4 av = *reinterpret_cast<const uint4 *>(ar + k);
                const uint4 bv = *reinterpret_cast<const uint4 *>(br + k);
                const uint32_t as[4] = {av.x, av.y, av.z, av.w}, bs[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t ai = inf_bytes<FMT_E5M2>(as[u]);
                    const uint32_t ns = (as[u] ^ bs[u]) & 0x80808080u;
                    bad |= ai & zero_bytes(bs[u]);
                    neg |= ai & ns;
                    pos |= ai & ~ns;
                }
            }
        }
        const uint32_t acc = (bad || (pos && neg)) ? kCanonNan32 : (neg ? 0xFF800000u : 0x7F800000u);
        const int64_t m = p.a_is_w ? b0 + r : a, n = p.a_is_w ? a : b0 + r;
        store_epilogue(p.out_kind, p.out, m * p.ldo + n, acc, alpha, sr);
    }
}

}  // namespace

hipError_t launch_inf_rows(const DeferParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)((p.ra + kRowWaves - 1) / kRowWaves);
    hipLaunchKernelGGL(inf_rows_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_inf_fixup(const DeferParams &p, hipStream_t stream)
{
    if (p.b_rows < 1 || p.b_rows > 16 || p.a_rows < 1 || (p.K + 16) * p.b_rows > kDeferLdsBytes)
        return hipErrorInvalidValue;
    const unsigned gx = (unsigned)((p.rb + p.b_rows - 1) / p.b_rows);
    const unsigned gy = (unsigned)((p.ra + p.a_rows - 1) / p.a_rows);
    if (gy > 65535u) return hipErrorInvalidValue;
    const size_t lds = (size_t)(p.K + 16) * p.b_rows;
    hipLaunchKernelGGL(inf_fixup_kernel, dim3(gx, gy), dim3(256), lds, stream, p);
    return hipGetLastError();
}

}  // namespace emu
