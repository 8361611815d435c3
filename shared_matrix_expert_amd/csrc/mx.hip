// The microscaling variant of the expert layer: MXFP4 shared and delta
// matrices on the scaled FP4 / FP8 matrix cores of gfx950.
//
// The pages ship 4-bit floating-point builds of the model (byteiota
// "Edge0-145B: Run a 145B Open-Source Model on Your Laptop", What You Need to
// Run It).  MI355X's native 4-bit format is MXFP4 (OCP Microscaling Formats:
// E2M1 elements, one E8M0 power-of-two scale per 32 along K), and its matrix
// cores multiply MXFP4 by MXFP8 (E4M3) directly, applying both operands' block
// scales themselves: v_mfma_scale_f32_16x16x128_f8f6f4.  So the large
// products (S_up and A_up with the token rows x, S_dn and A_dn with the
// activation rows a) take x and a quantised to MXFP8 along K.  The rank-r
// inputs z1, z2 (bf16 after R1, R4) meet B_up, B_dn unquantised: those
// matrices are converted exactly to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4
// with the block's power-of-two scale) for the bf16 matrix cores.  The LoRA
// branch, the bf16 roundings R1-R5 and the combine are the int4 layer's.
//
// Operand layouts of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on gfx950
// with random codes against a host product): lane l = 16 g + m.
//   A (E4M3, 8 VGPRs): row m; bytes 0-15 are K 16 g .. 16 g + 15, bytes 16-31
//     are K 64 + 16 g .. 64 + 16 g + 15.
//   B (E2M1, 4 VGPRs): column m; nibbles 0-31 are K 32 g .. 32 g + 31 (low
//     nibble first).
//   Scales: lane l's byte is the E8M0 of (row / column m, K block g).
//   D: as every 16 x 16 MFMA, rows 4 g .. 4 g + 3 of column m.
// Inside one instruction the products are summed with about 2^-13.5 of the
// terms' magnitude sum (measured), so these kernels meet the layer's
// tolerance through the bf16 roundings, not bit-for-bit.
//
// Kernels:
//   mx_quant      bf16 rows -> E4M3 codes + E8M0 scales (x)
//   mx_gemm<M>    the four large products, LDS-tiled:
//                   MX_Z1   z1 = R1(A_up Q(x))           per row (expert tiles)
//                   MX_HS   Hs = S_up Q(x) + V_up zl     per distinct (token, group)
//                   MX_Z2   z2 = R4(A_dn Q(a))           per row
//                   MX_OUT  o  = S_dn Q(a) + B_dn z2 + V_dn zl2   per row
//   mx_act        a = R3(SiLU(Hs + B_up z1)), written as bf16 and as Q(a)
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace em {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr float kE4M3Max = 448.0f;

// s_waitcnt with vmcnt = n and the other counters left free (gfx9 encoding).
template <int N>
EM_DEV void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// E8M0 byte of a block whose largest magnitude has bf16 bits m (sign cleared):
// floor(log2(amax)) - 8 + 127, limited to 0..254; 0 for an all-zero block.
EM_DEV int block_exp(uint32_t m) {
    if (m == 0) return 0;
    const int e8 = (int)(m >> 7);
    const int e = e8 ? e8 - 127 : (31 - __builtin_clz(m & 0x7Fu)) - 133;   // bf16 subnormal: mant * 2^-133
    return min(max(e - 8 + 127, 0), 254);
}

// Four bf16 values (two words) times 2^(127 - X), as E4M3 codes in one word
// (value 0 in byte 0).  The hardware conversion rounds to nearest even and
// turns magnitudes from 464 up into NaN, so the value is clamped to +-448
// first, which gives the saturating rounding.
EM_DEV uint32_t e4m3x4(uint32_t w0, uint32_t w1, float inv) {
    const float f0 = fminf(fmaxf(bf16_to_f32(w0 & 0xFFFFu) * inv, -kE4M3Max), kE4M3Max);
    const float f1 = fminf(fmaxf(bf16_to_f32(w0 >> 16) * inv, -kE4M3Max), kE4M3Max);
    const float f2 = fminf(fmaxf(bf16_to_f32(w1 & 0xFFFFu) * inv, -kE4M3Max), kE4M3Max);
    const float f3 = fminf(fmaxf(bf16_to_f32(w1 >> 16) * inv, -kE4M3Max), kE4M3Max);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, r, true);
    return (uint32_t)r;
}

EM_DEV float exp2_neg(int X) { return __uint_as_float((uint32_t)(254 - X) << 23); }   // 2^(127 - X)

// 32 MXFP4 weights of one block (16 bytes, element 2i in the low nibble of
// byte i) times their scale 2^(X - 127), exactly, as bf16 MFMA operands:
// out[s] holds elements 8 s .. 8 s + 7.  Exact while the products stay in
// bf16's range (scale bytes up to 252).
EM_DEV void fp4_block_bf16(const uint4& q, int X, uint4 (&out)[4]) {
    const float sc = __uint_as_float(X ? (uint32_t)X << 23 : 0x00400000u);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint32_t o[4];
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[s], sc, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[s], sc, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[s], sc, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[s], sc, 3));
        out[s] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

EM_DEV uint32_t amax16(const uint4& a, const uint4& b) {
    uint32_t m = 0;
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    return m;
}

}  // namespace

// ------------------------------------------------------------------ quantiser --
// One thread per block of 32 (64 bytes in, 32 + 1 out).  src rows are
// contiguous with K a multiple of 128, so block b (row b / nkb, block b % nkb)
// starts at element 32 b; its scale goes to the K-step-major array
// [K/128][rows][4].
__global__ void __launch_bounds__(256)
mx_quant(const uint16_t* __restrict__ src, int64_t rows, int nkb, uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const int64_t b = blockIdx.x * 256ll + threadIdx.x;
    if (b >= rows * nkb) return;
    const uint4* p = reinterpret_cast<const uint4*>(src + b * 32);
    const uint4 v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3];
    const int X = block_exp(max(amax16(v0, v1), amax16(v2, v3)));
    const float inv = exp2_neg(X);
    uint4* o = reinterpret_cast<uint4*>(q + b * 32);
    o[0] = make_uint4(e4m3x4(v0.x, v0.y, inv), e4m3x4(v0.z, v0.w, inv), e4m3x4(v1.x, v1.y, inv), e4m3x4(v1.z, v1.w, inv));
    o[1] = make_uint4(e4m3x4(v2.x, v2.y, inv), e4m3x4(v2.z, v2.w, inv), e4m3x4(v3.x, v3.y, inv), e4m3x4(v3.z, v3.w, inv));
    const int64_t row = b / nkb;
    const int kb = (int)(b % nkb);
    sc[((int64_t)(kb >> 2) * rows + row) * 4 + (kb & 3)] = (uint8_t)X;
}

// ------------------------------------------------------------------ the GEMM ---
namespace {

enum MxMode { MX_HS = 0, MX_OUT = 1, MX_Z1 = 2, MX_Z2 = 3 };
constexpr int MBM = 128, MBK = 128, MX_TH = 512;

// Waves are 2 (rows) x 4 (columns); each takes 64 rows x BN / 4 columns.  The
// shared products tile 512 columns, so that each activation tile read from
// the L2 feeds 512 columns, with three stages (loads two steps ahead); the
// rank-128 inputs tile their 128 columns with four stages.
template <int MODE>
struct MxCfg {
    static constexpr bool Z = MODE == MX_Z1 || MODE == MX_Z2;
    static constexpr int BN = Z ? 128 : 512;
    static constexpr int WN = BN / 4;
    static constexpr int NJ = WN / 16;
    static constexpr int NI = 4;
    static constexpr int A_B = MBM * MBK;          // E4M3 tile
    static constexpr int B_B = BN * (MBK / 2);     // E2M1 tile
    static constexpr int AS_B = MBM * 4, BS_B = BN * 4;
    static constexpr int STAGE = A_B + B_B + AS_B + BS_B;
    static constexpr int STAGES = Z ? 4 : 3;
    static constexpr int B_INSTR = BN / 16 / 8;    // 16-byte weight loads per wave per stage
    static constexpr int BS_W0 = Z ? 2 : 0;        // first wave of the BN / 64 weight-scale loads
};

struct MxTile { int g, r0, r1, n0; };

// Tile b: HS / OUT: row tiles of the groups in group order, columns fastest;
// Z1 / Z2: the experts' row tiles (one column tile), from the per-expert
// 128-row tile prefix.
template <int MODE>
EM_DEV bool mx_tile(const LayerArgs& a, int b, int ntn, MxTile& t) {
    if constexpr (MxCfg<MODE>::Z) {
        const int32_t* tp = a.db.etile_pf;
        if (b >= tp[a.E]) return false;
        int lo = 0, hi = a.E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tp[mid] <= b) lo = mid; else hi = mid;
        }
        t.g = lo;
        t.r0 = a.db.eoff[lo] + (b - tp[lo]) * MBM;
        t.r1 = min(a.db.eoff[lo + 1], t.r0 + MBM);
        t.n0 = 0;
        return true;
    }
    int m = b / ntn;
    t.n0 = (b % ntn) * MxCfg<MODE>::BN;
    for (int g = 0; g < a.G; ++g) {
        const int r0 = MODE == MX_HS ? a.db.uoff[g] : a.db.eoff[g * a.P];
        const int r1 = MODE == MX_HS ? a.db.uoff[g + 1] : a.db.eoff[(g + 1) * a.P];
        const int nt = (r1 - r0 + MBM - 1) / MBM;
        if (m < nt) {
            t.g = g;
            t.r0 = r0 + m * MBM;
            t.r1 = min(r1, t.r0 + MBM);
            return true;
        }
        m -= nt;
    }
    return false;
}

// Per-thread DMA sources for the whole K range.
//   A: round q (0, 1) of wave w covers tile rows 8 (2 w + q) .. + 7; lane l
//      writes LDS slot l % 8 of row 8 (2 w + q) + l / 8 and fetches that row's
//      16-byte segment (l % 8) ^ ((row >> 1) & 7), so that the fragment reads
//      (16 rows, one segment each) fall on 16 distinct bank groups.
//   B: round q of wave w covers columns 16 (B_INSTR w + q) .. + 15; lane l
//      writes slot l % 4 of column 16 (..) + l / 4, fetching segment
//      (l % 4) ^ ((col >> 2) & 3).
//   Scales (stored K-step-major, [K/128][rows][4], so one step's words of
//      consecutive rows are consecutive): waves 0, 1 fetch the A rows' words;
//      waves BS_W0 .. BS_W0 + BN / 64 - 1 the B columns'.
template <int MODE>
struct MxSrc {
    const uint8_t* a[2];     // A row (with segment) per round, at K = 0
    const uint8_t* b[MxCfg<MODE>::B_INSTR];
    const uint8_t* as;       // A-scale word of this lane at K step 0 (waves 0, 1), else null
    const uint8_t* bs;       // B-scale word of this lane at K step 0, or null
    size_t as_step, bs_step; // bytes between K steps
};

template <int MODE>
EM_DEV void mx_fetch(uint8_t* stage, const MxSrc<MODE>& src, int ks) {
    using C = MxCfg<MODE>;
    const int w = wave_id();
    uint8_t* As = stage;
    uint8_t* Bs = stage + C::A_B;
    uint8_t* AS = Bs + C::B_B;
    uint8_t* BS = AS + C::AS_B;
#pragma unroll
    for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.a[q] + (size_t)ks * MBK),
                                         (lds_ptr_t)(As + (8 * (2 * w + q)) * MBK), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < C::B_INSTR; ++q)
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.b[q] + (size_t)ks * (MBK / 2)),
                                         (lds_ptr_t)(Bs + 16 * (C::B_INSTR * w + q) * (MBK / 2)), 16, 0, 0);
    if (src.as)
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.as + ks * src.as_step), (lds_ptr_t)(AS + 256 * w), 4, 0, 0);
    if (src.bs)
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.bs + ks * src.bs_step),
                                         (lds_ptr_t)(BS + 256 * (w - C::BS_W0)), 4, 0, 0);
}

template <int MODE>
EM_DEV void mx_compute(floatx4 (&acc)[MxCfg<MODE>::NI][MxCfg<MODE>::NJ], const uint8_t* stage) {
    using C = MxCfg<MODE>;
    const int l = lane_id(), g = l >> 4, m = l & 15;
    const int wv = wave_id(), wm = wv >> 2, wn = wv & 3;
    const uint8_t* As = stage;
    const uint8_t* Bs = stage + C::A_B;
    const uint32_t* AS = reinterpret_cast<const uint32_t*>(Bs + C::B_B);
    const uint32_t* BS = reinterpret_cast<const uint32_t*>(Bs + C::B_B + C::AS_B);
    v8i bf[C::NJ];
    int sb[C::NJ];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
        const int col = C::WN * wn + 16 * j + m;
        const uint4 v = *reinterpret_cast<const uint4*>(Bs + col * (MBK / 2) + 16 * (g ^ ((col >> 2) & 3)));
        bf[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sb[j] = (int)__builtin_amdgcn_ubfe(BS[col], 8 * g, 8);
    }
    auto frag = [&](int i, v8i& af, int& sa) {
        const int row = 64 * wm + 16 * i + m;
        const int sw = (row >> 1) & 7;
        const uint4 lo = *reinterpret_cast<const uint4*>(As + row * MBK + 16 * (g ^ sw));
        const uint4 hi = *reinterpret_cast<const uint4*>(As + row * MBK + 16 * ((4 + g) ^ sw));
        af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sa = (int)__builtin_amdgcn_ubfe(AS[row], 8 * g, 8);
    };
    v8i afc, afn;
    int sac, san;
    frag(0, afc, sac);
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
        if (i + 1 < C::NI) frag(i + 1, afn, san);
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afc, bf[j], acc[i][j], 0, 4, 0, sac, 0, sb[j]);
        afc = afn;
        sac = san;
    }
}

// Wait until at most `n` of this wave's loads are in flight (n is one of the
// few values the pipeline produces).
EM_DEV void wait_vm_n(int n) {
    switch (n) {
        case 0: wait_vm<0>(); break;
        case 3: wait_vm<3>(); break;
        case 4: wait_vm<4>(); break;
        case 5: wait_vm<5>(); break;
        case 6: wait_vm<6>(); break;
        case 7: wait_vm<7>(); break;
        case 8: wait_vm<8>(); break;
        case 10: wait_vm<10>(); break;
        default: wait_vm<0>(); break;
    }
}

}  // namespace

template <int MODE>
__global__ void __launch_bounds__(MX_TH)
mx_gemm(LayerArgs a) {
    using C = MxCfg<MODE>;
    constexpr int BN = C::BN, WN = C::WN, NI = C::NI, NJ = C::NJ;
    constexpr int STAGES = C::STAGES;
    __shared__ __attribute__((aligned(16))) uint8_t lds[STAGES * C::STAGE];
    const int ntn = C::Z ? 1 : (MODE == MX_HS ? a.h : a.d) / BN;
    // XCD-aware order: XCD x = blockIdx % 8 takes tiles [x * per, (x + 1) * per)
    const int per = gridDim.x >> 3;
    const int b = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    MxTile t;
    if (!mx_tile<MODE>(a, b, ntn, t)) return;

    const int K = (MODE == MX_HS || MODE == MX_Z1) ? a.d : a.h;
    const int N = C::Z ? a.r : (MODE == MX_HS ? a.h : a.d);
    const uint8_t* W = MODE == MX_HS ? a.s_up : (MODE == MX_OUT ? a.s_dn : (MODE == MX_Z1 ? a.a_up : a.a_dn));
    const uint8_t* WE = MODE == MX_HS ? a.s_up_e : (MODE == MX_OUT ? a.s_dn_e : (MODE == MX_Z1 ? a.a_up_e : a.a_dn_e));
    const uint8_t* AQ = (MODE == MX_HS || MODE == MX_Z1) ? a.xq : a.aq;
    const uint8_t* AE = (MODE == MX_HS || MODE == MX_Z1) ? a.xs : a.as;
    const int l = lane_id(), wv = wave_id(), g = l >> 4, m = l & 15;
    const int nrow = t.r1 - t.r0;

    // A row of a tile row (rows past the tile's end repeat its last row)
    auto a_row = [&](int tr) -> int64_t {
        const int r = t.r0 + min(tr, nrow - 1);
        if constexpr (MODE == MX_HS) return a.db.ut_tok[r];
        else if constexpr (MODE == MX_Z1) return a.db.row_tok[r];
        else return r;
    };
    MxSrc<MODE> src;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tr = 8 * (2 * wv + q) + (l >> 3);
        src.a[q] = AQ + a_row(tr) * K + 16 * ((l & 7) ^ ((tr >> 1) & 7));
    }
    const uint8_t* Wt = W + ((size_t)t.g * N + t.n0) * (K / 2);
#pragma unroll
    for (int q = 0; q < C::B_INSTR; ++q) {
        const int col = 16 * (C::B_INSTR * wv + q) + (l >> 2);
        src.b[q] = Wt + (size_t)col * (K / 2) + 16 * ((l & 3) ^ ((col >> 2) & 3));
    }
    // scale words: activations [K/128][rows][4] (rows of x for HS / Z1, of a
    // for Z2 / OUT), weights [lead][K/128][N][4]
    const int64_t a_rows = (MODE == MX_HS || MODE == MX_Z1) ? a.T : a.rmax;
    src.as = wv < 2 ? AE + a_row(64 * wv + l) * 4 : nullptr;
    src.as_step = (size_t)a_rows * 4;
    const int bsw = wv - C::BS_W0;
    src.bs = (bsw >= 0 && bsw < BN / 64) ? WE + ((size_t)t.g * (K / 128) * N + t.n0 + 64 * bsw + l) * 4 : nullptr;
    src.bs_step = (size_t)N * 4;
    const int per_stage = 2 + C::B_INSTR + (src.as ? 1 : 0) + (src.bs ? 1 : 0);   // this wave's loads per stage

    floatx4 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();
    // The LoRA and per-expert delta products go into the accumulators before
    // the main loop: every load they make is consumed before the first
    // stage's, and the main loop's operand state is not yet live, so the
    // epilogue is left with the stores alone.
    if constexpr (!C::Z) {
        const int wm = wv >> 2, wn = wv & 3;
        // ---- LoRA branch: V[g] (bf16 [N][rL]) x the rounded LoRA input rows (bf16 [rows][rLp])
        const int rLp = (a.rL + 7) & ~7;
        {
            const uint16_t* V = (MODE == MX_HS ? a.lu_v : a.ld_v) + (size_t)t.g * N * a.rL;
            const uint16_t* Zl = MODE == MX_HS ? a.zl : a.zl2;
            for (int kb = 0; kb < a.rL; kb += 32) {
                const bool kv = kb + 8 * g < a.rL;
                uint4 bv[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int n = t.n0 + WN * wn + 16 * j + m;
                    bv[j] = kv ? ld16(V + (size_t)n * a.rL + kb + 8 * g) : zero_u4();
                }
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int row = t.r0 + min(64 * wm + 16 * i + m, nrow - 1);
                    const uint4 av = kv ? ld16(Zl + (size_t)row * rLp + kb + 8 * g) : zero_u4();
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_bf16(av, bv[j], acc[i][j]);
                }
            }
        }

        // ---- per-expert delta down: B_dn[e] (MXFP4 [d][r], exact in bf16) x z2 rows of expert e.
        // Lane group g takes K block g (32 elements): its 16 code bytes and scale
        // convert to the four bf16 operands of steps s = 0..3 (elements 8 s ..).
        if constexpr (MODE == MX_OUT) {
            const int e_first = a.db.row_exp[t.r0], e_last = a.db.row_exp[t.r1 - 1];
            for (int e = e_first; e <= e_last; ++e) {
                const int p = max(a.db.eoff[e], t.r0) - t.r0;          // tile rows [p, q) are expert e's
                const int q = min(a.db.eoff[e + 1], t.r1) - t.r0;
                if (p >= q) continue;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int rl = 64 * wm + 16 * i;                    // subtile rows [rl, rl + 16)
                    if (rl + 16 <= p || rl >= q) continue;              // wave-uniform
                    const int row = rl + m;
                    const bool mine = row >= p && row < q;
                    const uint16_t* zr = a.z2 + (size_t)(t.r0 + (mine ? row : p)) * KC + 32 * g;
                    uint4 af[4];
#pragma unroll
                    for (int st = 0; st < 4; ++st) af[st] = mine ? ld16(zr + 8 * st) : zero_u4();
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {                      // one column subtile's operands at a time
                        uint4 bq[4];
                        const size_t n = (size_t)e * a.d + t.n0 + WN * wn + 16 * j + m;
                        fp4_block_bf16(ld16(a.b_dn + n * (KC / 2) + 16 * g), a.b_dn_e[n * (KC / 32) + g], bq);
#pragma unroll
                        for (int st = 0; st < 4; ++st) acc[i][j] = mfma_bf16(af[st], bq[st], acc[i][j]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    }

    // ---- main loop: loads STAGES - 1 K steps ahead of the math
    const int nk = K / MBK;
    for (int s = 0; s < STAGES - 1 && s < nk; ++s) mx_fetch<MODE>(lds + s * C::STAGE, src, s);
    wait_vm_n(per_stage * (min(nk, STAGES - 1) - 1));
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int ahead = ks + STAGES - 1;
        if (ahead < nk) mx_fetch<MODE>(lds + (ahead % STAGES) * C::STAGE, src, ahead);
        mx_compute<MODE>(acc, lds + (ks % STAGES) * C::STAGE);
        // the next step's loads must have landed: the later ones may stay in flight
        const int later = min(nk - 1, ks + STAGES - 1) - (ks + 1);
        wait_vm_n(per_stage * max(later, 0));
        __syncthreads();
    }

    const int wm = wv >> 2, wn = wv & 3;
    // ---- R1 / R4 inputs: rounded to bf16
    if constexpr (C::Z) {
        uint16_t* out = MODE == MX_Z1 ? a.z1 : a.z2;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tr = 64 * wm + 16 * i + 4 * g + v;
                if (tr >= nrow) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    out[(size_t)(t.r0 + tr) * a.r + WN * wn + 16 * j + m] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
            }
        return;
    }

    // ---- store: lane holds rows 16 i + 4 g + v of its wave's 64, column 16 j + m of its wave's block
    float* out = MODE == MX_HS ? a.hs : a.o;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tr = 64 * wm + 16 * i + 4 * g + v;
            if (tr >= nrow) continue;
            float* orow = out + (size_t)(t.r0 + tr) * N + t.n0 + WN * wn + m;
#pragma unroll
            for (int j = 0; j < NJ; ++j) orow[16 * j] = acc[i][j][v];
        }
}

// ------------------------------------------------------------------ activation --
// a[row] = R3(SiLU(Hs[u(row)] + B_up[e] z1[row])) for a 64-row task of
// expert e and 256 columns (r = 128; B_up converted exactly to bf16, lane
// group g taking K block g), written as bf16 and as Q(a): each thread owns
// one row's 16 columns, the two threads of a 32-column block exchange their
// maxima.
__global__ void __launch_bounds__(256)
mx_act(LayerArgs a) {
    __shared__ float ot[64][64 + 4];
    const int b = blockIdx.x;
    const int s_e = [&] {
        const int32_t* tiles = a.db.etile;
        if (b >= tiles[a.E]) return -1;
        int lo = 0, hi = a.E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tiles[mid] <= b) lo = mid; else hi = mid;
        }
        return lo;
    }();
    if (s_e < 0) return;
    const int rbeg = a.db.eoff[s_e] + (b - a.db.etile[s_e]) * 64;
    const int rows = min(a.db.eoff[s_e + 1] - rbeg, 64);
    if (rows <= 0) return;
    const int l = lane_id(), wv = wave_id(), g = l >> 4, m = l & 15;
    const int n0 = blockIdx.y * 256;

    uint4 af[4][4];                                      // z1 rows: af[ms][s] = elements 32 g + 8 s ..
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
        const size_t r = rbeg + min(16 * ms + m, rows - 1);
#pragma unroll
        for (int st = 0; st < 4; ++st) af[ms][st] = ld16(a.z1 + r * KC + 32 * g + 8 * st);
    }
    const int tr = threadIdx.x >> 2, tq = threadIdx.x & 3;   // epilogue: row, 16-column quarter
    const int u = tr < rows ? a.db.row_u[rbeg + tr] : 0;
    for (int cb = 0; cb < 4; ++cb) {
        const size_t n = (size_t)s_e * a.h + n0 + 64 * cb + 16 * wv + m;
        uint4 bq[4];
        fp4_block_bf16(ld16(a.b_up + n * (KC / 2) + 16 * g), a.b_up_e[n * (KC / 32) + g], bq);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
            floatx4 acc = zero4();
#pragma unroll
            for (int st = 0; st < 4; ++st) acc = mfma_bf16(af[ms][st], bq[st], acc);
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) ot[16 * ms + 4 * g + vv][16 * wv + m] = acc[vv];
        }
        __syncthreads();
        // every thread takes part in the pair exchange (rows past the task's
        // end work on a zero row and store nothing)
        const int col = n0 + 64 * cb + 16 * tq;
        uint32_t ob[8];
        {
            const bool live = tr < rows;
            const float4* hp = reinterpret_cast<const float4*>(a.hs + (size_t)u * a.h + col);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 hv = live ? hp[q] : make_float4(0.f, 0.f, 0.f, 0.f);
                const float* o = &ot[tr][16 * tq + 4 * q];
                const uint32_t b0 = f32_to_bf16_rne(silu(o[0] + hv.x));
                const uint32_t b1 = f32_to_bf16_rne(silu(o[1] + hv.y));
                const uint32_t b2 = f32_to_bf16_rne(silu(o[2] + hv.z));
                const uint32_t b3 = f32_to_bf16_rne(silu(o[3] + hv.w));
                ob[2 * q] = b0 | (b1 << 16);
                ob[2 * q + 1] = b2 | (b3 << 16);
            }
        }
        const uint4 w0 = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        const uint4 w1 = make_uint4(ob[4], ob[5], ob[6], ob[7]);
        const uint32_t mine = amax16(w0, w1);
        const uint32_t other = (uint32_t)__shfl_xor((int)mine, 1, 64);
        const int X = block_exp(max(mine, other));
        const float inv = exp2_neg(X);
        if (tr < rows) {
            const size_t row = (size_t)(rbeg + tr);
            uint4* ap = reinterpret_cast<uint4*>(a.act + row * a.h + col);
            ap[0] = w0;
            ap[1] = w1;
            *reinterpret_cast<uint4*>(a.aq + row * a.h + col) =
                make_uint4(e4m3x4(w0.x, w0.y, inv), e4m3x4(w0.z, w0.w, inv), e4m3x4(w1.x, w1.y, inv),
                           e4m3x4(w1.z, w1.w, inv));
            if ((tq & 1) == 0) a.as[((size_t)(col >> 7) * a.rmax + row) * 4 + ((col >> 5) & 3)] = (uint8_t)X;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ host side ---

bool mx_layer_ok(int d, int h, int r, int rL) {
    return r == KC && d % 512 == 0 && h % 512 == 0 && rL % 8 == 0 && rL >= 8 && rL <= 32;
}

static hipError_t launch_quant(const uint16_t* src, int64_t rows, int K, uint8_t* q, uint8_t* sc, hipStream_t s,
                               const char* name) {
    const int64_t nblk = rows * (K / 32);
    if (nblk == 0) return hipSuccess;
    prof_begin(s);
    mx_quant<<<(unsigned)((nblk + 255) / 256), 256, 0, s>>>(src, rows, K / 32, q, sc);
    prof_end(s, name);
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemm_mx(const LayerArgs& a, int64_t max_rows, hipStream_t s, const char* name) {
    int64_t blocks;
    if constexpr (MxCfg<MODE>::Z) {
        blocks = max_rows / MBM + (a.E < max_rows ? a.E : max_rows) + 1;   // >= sum over experts of ceil(rows_e / BM)
    } else {
        const int ntn = (MODE == MX_HS ? a.h : a.d) / MxCfg<MODE>::BN;
        blocks = (max_rows / MBM + a.G + 1) * ntn;                         // >= sum over groups of ceil(rows_g / BM)
    }
    blocks = (blocks + 7) & ~7ll;
    prof_begin(s);
    mx_gemm<MODE><<<(unsigned)blocks, MX_TH, 0, s>>>(a);
    prof_end(s, name);
    return hipGetLastError();
}

// The layer after the dispatch kernels: every stage of the MX variant.
hipError_t launch_mx_layer(const LayerArgs& a, hipStream_t s) {
    hipError_t e = launch_quant(a.x, a.T, a.d, a.xq, a.xs, s, "mx_quant_x");
    if (e == hipSuccess) e = launch_gemm_mx<MX_Z1>(a, a.rmax, s, "mx_z1");
    if (e != hipSuccess) return e;
    launch_lora_in(a, 0, s);
    e = launch_gemm_mx<MX_HS>(a, a.umax, s, "mx_shared_up");
    if (e != hipSuccess) return e;
    prof_begin(s);
    mx_act<<<dim3(a.max_etiles, a.h / 256), 256, 0, s>>>(a);
    prof_end(s, "mx_act");
    e = launch_gemm_mx<MX_Z2>(a, a.rmax, s, "mx_z2");
    if (e != hipSuccess) return e;
    launch_lora_in(a, 1, s);
    e = launch_gemm_mx<MX_OUT>(a, a.rmax, s, "mx_down");
    if (e != hipSuccess) return e;
    return launch_combine(a, s);
}

}  // namespace em
