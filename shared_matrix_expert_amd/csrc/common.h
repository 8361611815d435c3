// Device helpers shared by the layer's kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define EM_DEV __device__ __forceinline__

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace em {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 / fp16 ----

EM_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round a finite float to bf16, nearest-even.
EM_DEV uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

EM_DEV float fp16_bits_to_f32(uint16_t b) {
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}

// ---------------------------------------------------------------- int4 dequant ----
// A packed dword holds 8 signed nibbles, element 2i in the low nibble of byte i
// and 2i+1 in the high nibble.  v_cvt_off_f32_i4 turns the low nibble of its
// (SDWA-selected) source byte into q/16 as an exact float; the high nibbles go
// through the same instruction after a 4-bit shift.  q/16 has at most 4
// significant bits, so its bf16 is the float's upper half taken without
// rounding, and two of them pack into one dword with a byte permute.  The
// factor 1/16 is returned to the result through the group scale (x16, exact).
#define EM_CVT_OFF(OUT, SRC, SEL)                                                   \
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD " \
                 "src0_sel:" SEL                                                    \
                 : "=v"(OUT)                                                        \
                 : "v"(SRC))

// out[i] = { bf16(q[2i]/16) | bf16(q[2i+1]/16) << 16 } for i = 0..3 (elements
// in their natural order, so the dword is a ready MFMA operand pair).
EM_DEV void dequant8(uint32_t w, uint32_t out[4]) {
    uint32_t w4 = w >> 4;
    float e0, e1, e2, e3, e4, e5, e6, e7;
    EM_CVT_OFF(e0, w, "BYTE_0");
    EM_CVT_OFF(e2, w, "BYTE_1");
    EM_CVT_OFF(e4, w, "BYTE_2");
    EM_CVT_OFF(e6, w, "BYTE_3");
    EM_CVT_OFF(e1, w4, "BYTE_0");
    EM_CVT_OFF(e3, w4, "BYTE_1");
    EM_CVT_OFF(e5, w4, "BYTE_2");
    EM_CVT_OFF(e7, w4, "BYTE_3");
    out[0] = __builtin_amdgcn_perm(__float_as_uint(e1), __float_as_uint(e0), 0x07060302u);
    out[1] = __builtin_amdgcn_perm(__float_as_uint(e3), __float_as_uint(e2), 0x07060302u);
    out[2] = __builtin_amdgcn_perm(__float_as_uint(e5), __float_as_uint(e4), 0x07060302u);
    out[3] = __builtin_amdgcn_perm(__float_as_uint(e7), __float_as_uint(e6), 0x07060302u);
}

// ---------------------------------------------------------------- MFMA ----------
// D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Operand lane layout: lane l supplies row (A) / column (B) l % 16 and the
// eight K-elements of slot l / 16; the result lane l holds D[4*(l/16)+v][l%16].
EM_DEV floatx4 mfma_bf16(uint4 a, uint4 b, floatx4 c) {
    bf16x8 av = __builtin_bit_cast(bf16x8, a);
    bf16x8 bv = __builtin_bit_cast(bf16x8, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

EM_DEV floatx4 zero4() { floatx4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// acc + s * t, one fused multiply-add per element (a scaled chunk sum added to
// its accumulator with a single rounding).
EM_DEV floatx4 fma4(float s, floatx4 t, floatx4 acc) {
    floatx4 r;
    r.x = __builtin_fmaf(s, t.x, acc.x);
    r.y = __builtin_fmaf(s, t.y, acc.y);
    r.z = __builtin_fmaf(s, t.z, acc.z);
    r.w = __builtin_fmaf(s, t.w, acc.w);
    return r;
}

// ---------------------------------------------------------------- misc ----------
EM_DEV int lane_id() { return threadIdx.x & (kWave - 1); }
// The wave's index in the workgroup, in a scalar register: the compiler cannot
// see on its own that it is uniform across the wave, and loops bounded by it
// would otherwise be compiled as divergent loops.
EM_DEV int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// SiLU(v) = v / (1 + e^-v) from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32, each within about 1 ulp): a few fp32 ulps from the
// exact value, far inside the bf16 rounding that follows it.
EM_DEV float silu(float v) {
    const float e = __builtin_amdgcn_exp2f(-v * 1.4426950408889634f);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// An 8-byte global store that the compiler's wait insertion does not see.
// Loads and stores share one counter on this target, and a counted store in
// flight makes the compiler wait for zero before the next use of any load.
// Loads complete in order among themselves, so a store it does not count can
// only lengthen a vmcnt(N) wait, never end it early.  For results that
// nothing in the same launch reads back; the launch's end makes them visible.
EM_DEV void st8_uncounted(void* p, uint64_t v) {
    asm volatile("global_store_dwordx2 %0, %1, off" : : "v"(p), "v"(v) : "memory");
}

}  // namespace em
