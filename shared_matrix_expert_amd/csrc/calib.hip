// Calibration kernel: the measured rate of the matrix cores, to set beside the
// published dense bf16 peak.  Not a step of the layer.
#include "common.h"
#include "kernels.h"

namespace em {

// Every wave runs `iters` rounds of eight independent chains of
// v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 x 2 = 16384 flops each) on register
// operands; the accumulators are folded into one store per lane so that no
// chain can be dropped.
__global__ void __launch_bounds__(256)
mfma_peak(float* __restrict__ out, int iters) {
    const uint32_t one = 0x3F803F80u;                                  // bf16 pair (1, 1)
    const uint32_t tiny = 0x2F802F80u | (threadIdx.x & 1u);            // bf16 pair near 2^-32
    const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(one, one, one, one));
    const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(tiny, tiny, tiny, tiny));
    // eight independent accumulators, each one product per round; the product
    // is written out so that the compiler keeps every accumulator in its own
    // registers (left to itself it rotates them through register moves around
    // the loop, and every move waits on a product)
    floatx4 c0 = zero4(), c1 = zero4(), c2 = zero4(), c3 = zero4();
    floatx4 c4 = zero4(), c5 = zero4(), c6 = zero4(), c7 = zero4();
    for (int it = 0; it < iters; ++it) {
        // the compiler does not see the products inside the asm, so the block
        // waits out vector writes of its operands itself
        asm volatile(
            "s_nop 2\n\t"
            "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
            "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
            "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
            "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
            "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
            "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
            "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
            : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
            : "v"(a), "v"(b));
    }
    // the last products are read only after the dependency wait on them
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7));
    const floatx4 s4 = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = (s4.x + s4.y) + (s4.z + s4.w);
}

hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t s) {
    prof_begin(s);
    mfma_peak<<<blocks, 256, 0, s>>>(out, iters);
    prof_end(s, "mfma_peak");
    return hipGetLastError();
}

}  // namespace em
