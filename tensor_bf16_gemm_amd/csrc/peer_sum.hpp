// peer_sum.hpp -- the reduction step of the unfused baseline: a separate,
// HBM-bound kernel that adds R-1 peer partials to a local bf16 product.
//
// The unfused pipeline the fused kernel is measured against (the GEMM-AR
// page's reference: the local matmul rounded to bf16, then the collective)
// runs a library GEMM and then this kernel: out = bf16(local + sum of the
// partials), summed in fp32 in the order local, peer 0, peer 1, ..., rounded
// to nearest-even once.  Every element is read and written once, so the
// kernel streams: 16 bytes (8 bf16) per lane per step, non-temporal loads and
// stores, all 1 + NP loads of a step issued before the adds.
#pragma once

#include "gc_kernel.hpp"

namespace gc {

constexpr int PS_THREADS = 256;

// out[e] = bf16(local[e] + sum_p partials[p * stride + e]), e in [0, n).
// local, partials, out 16-byte aligned and stride a multiple of 8 (checked
// by the host).
template <int NP>
__global__ __launch_bounds__(PS_THREADS) void peer_sum_kernel(const uint16_t *local,
                                                              const uint16_t *partials,
                                                              int64_t stride, int64_t n,
                                                              uint16_t *out)
{
    const int64_t nv = n / 8;
    const int64_t step = (int64_t)gridDim.x * PS_THREADS;
    for (int64_t v = (int64_t)blockIdx.x * PS_THREADS + threadIdx.x; v < nv; v += step) {
        u32x4_t x[NP + 1];
        x[0] = __builtin_nontemporal_load((const u32x4_t *)local + v);
#pragma unroll
        for (int p = 0; p < NP; ++p)
            x[p + 1] = __builtin_nontemporal_load((const u32x4_t *)(partials + p * stride) + v);
        f32x4_t lo = unpack_bf16x4((u32x2_t){x[0][0], x[0][1]});
        f32x4_t hi = unpack_bf16x4((u32x2_t){x[0][2], x[0][3]});
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            lo += unpack_bf16x4((u32x2_t){x[p + 1][0], x[p + 1][1]});
            hi += unpack_bf16x4((u32x2_t){x[p + 1][2], x[p + 1][3]});
        }
        const u32x2_t a = pack_bf16x4(lo), b = pack_bf16x4(hi);
        __builtin_nontemporal_store((u32x4_t){a[0], a[1], b[0], b[1]}, (u32x4_t *)out + v);
    }
    // the last n % 8 elements, one per lane of workgroup 0
    const int64_t e = nv * 8 + threadIdx.x;
    if (blockIdx.x == 0 && e < n) {
        float s = __uint_as_float((uint32_t)local[e] << 16);
        for (int p = 0; p < NP; ++p)
            s += __uint_as_float((uint32_t)partials[p * stride + e] << 16);
        out[e] = __builtin_bit_cast(uint16_t, (__bf16)s);
    }
}

}  // namespace gc
