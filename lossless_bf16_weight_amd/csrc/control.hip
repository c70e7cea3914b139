// Bandwidth control for the decode: a kernel that moves the bytes of a
// decode -- one read of a source region, one write of an output region of a
// different size -- with the same kind of accesses (16-byte non-temporal
// loads and stores, contiguous ranges per workgroup) and no decoding.  Its
// rate is the HBM ceiling the decoder can be held against, in the spirit of
// the control condition of the mlx-dfloat project page's overhead benchmark
// (the same path with the decoding taken out, so that the gap measures the
// decode).
#include <hip/hip_runtime.h>

#include "df11_internal.hpp"

namespace df11 {

typedef uint32_t c32x4 __attribute__((ext_vector_type(4)));

// Output unit i (16 bytes) is source unit floor(i * ratio) xor-ed with i:
// with ratio <= 1 (the host refuses a source larger than the output) every
// source unit is read, consecutive outputs sharing or advancing their source
// unit, and every output unit is written once.  Workgroups sweep the
// output in interleaved 32 KiB tiles (8 units per lane in flight), the order
// that measured fastest for this mix of reads and writes.
constexpr int kUnroll = 8;
__global__ __launch_bounds__(256) void bw_control_kernel(const c32x4 *src, uint64_t src16,
                                                         c32x4 *dst, uint64_t dst16, uint64_t ratio20) {
    for (uint64_t b = (uint64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; b < dst16;
         b += (uint64_t)gridDim.x * 256 * kUnroll) {
        c32x4 v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const uint64_t i = b + 256 * k;
            uint64_t s = (i * ratio20) >> 20;
            s = s < src16 ? s : src16 - 1;
            if (i < dst16) v[k] = __builtin_nontemporal_load(src + s);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const uint64_t i = b + 256 * k;
            if (i < dst16) {
                v[k].x ^= (uint32_t)i;
                __builtin_nontemporal_store(v[k], dst + i);
            }
        }
    }
}

hipError_t launch_bw_control(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes,
                             int grid, hipStream_t stream) {
    const uint64_t src16 = src_bytes / 16, dst16 = dst_bytes / 16;
    // ratio in 20-bit fixed point; i * ratio stays below 2^64 for the sizes
    // the host allows (dst16 < 2^36, ratio < 2^26)
    const uint64_t ratio20 = (src16 << 20) / dst16;
    hipLaunchKernelGGL(bw_control_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const c32x4 *>(src), src16, reinterpret_cast<c32x4 *>(dst), dst16,
                       ratio20);
    return hipGetLastError();
}

}  // namespace df11
