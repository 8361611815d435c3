// Shared-matrix products of large batches (steps a4 and a8-a10): LDS-tiled
// int4 x bf16 GEMMs on the matrix cores.
//
// Every group of 64 experts shares one up and one down matrix (launch post
// "Edge0-145B: Frontier AI Capabilities on Your Own Computer", Under the Hood,
// Architecture paragraph), so a prefill batch turns the shared part of the
// layer into one dense GEMM per group and matrix: the group's distinct tokens
// times S_up (up), the group's rows times S_dn (down).  At 16K tokens these
// two GEMMs are ~95 % of the layer's flops.
//
// Tile: 128 rows x 256 columns per workgroup of 8 waves (each wave all 128
// rows x its own 32 columns = 8 x 2 MFMA 16x16 subtiles; two waves per SIMD,
// so one wave's dequantisation and scaling overlap the other's matrix work,
// and every column is dequantised once per workgroup), K in steps of 128 = one
// quant group.  The activation tile (128 x 128 bf16 = 32 KB) and the
// weight tile (256 columns x 128 int4 = 16 KB) move from global memory
// straight into LDS (global_load_lds_dwordx4, no registers), three buffer sets
// deep so that every step's loads have two steps of math to arrive in; the
// 16-byte slots are XOR-swizzled so that the MFMA fragment reads are free of
// bank conflicts.  Each wave converts its 64 columns exactly to bf16 in
// registers; every 128-element chunk is accumulated in a fresh fp32 tile and
// added to the result times 16 x its fp16 scale, so the weight values are
// exactly q x s.
//
// Workgroup order: blockIdx is remapped so that each XCD (blockIdx mod 8) runs
// a contiguous range of tiles, columns fastest: the workgroups that share an
// activation tile run together on one XCD and read it from that XCD's L2.
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace em {

namespace {

constexpr int BM = kPfTileRows, BK = 128;
constexpr int PF_WAVES = 8, PF_TH = 64 * PF_WAVES;
constexpr int SLOTS = BK / 8;                    // 16-byte slots per activation row
constexpr int NI = BM / 16;                      // 16-row subtiles per wave (all BM rows)
static_assert(BM <= kPfSpareRows, "the last row tile reads up to BM - 1 rows past the end");

// Per mode: the shared products (HS, OUT) tile 256 columns, the rank-128
// inputs of the deltas (Z1 = A_up x, Z2 = A_dn a) their 128; each wave takes
// WN = BN / 8 columns of all BM rows.
template <int MODE>
struct PfCfg {
    static constexpr bool Z = MODE == PF_Z1 || MODE == PF_Z2;
    static constexpr int BN = Z ? 128 : 256;
    static constexpr int WN = BN / PF_WAVES;     // columns per wave (wave w: columns WN w)
    static constexpr int NJ = WN / 16;           // 16-column subtiles per wave
    static constexpr int STEP_VM = NJ + BN / 128 + BM / 32;   // vector-memory instructions per step
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// s_waitcnt with vmcnt = n and the other counters left free (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct PfTile {
    int g;          // group (HS, OUT) or expert (Z1, Z2)
    int r0, r1;     // rows [r0, r1) of the tile (r1 - r0 <= BM)
    int n0;         // first output column
};

// Tile b of the launch.  HS, OUT: row tiles of the groups in group order,
// columns fastest.  Z1, Z2: the experts' row tiles in expert order (one column
// tile), found by bisecting the per-expert tile prefix.
template <int MODE>
EM_DEV bool pf_tile(const LayerArgs& a, int b, int ntn, PfTile& t) {
    if constexpr (PfCfg<MODE>::Z) {
        const int32_t* tp = a.db.etile_pf;
        if (b >= tp[a.E]) return false;
        int lo = 0, hi = a.E;                    // tp[lo] <= b < tp[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tp[mid] <= b) lo = mid;
            else hi = mid;
        }
        t.g = lo;
        t.r0 = a.db.eoff[lo] + (b - tp[lo]) * BM;
        t.r1 = min(a.db.eoff[lo + 1], t.r0 + BM);
        t.n0 = 0;
        return true;
    }
    int m = b / ntn;
    t.n0 = (b % ntn) * PfCfg<MODE>::BN;
    for (int g = 0; g < a.G; ++g) {
        const int r0 = MODE == PF_HS ? a.db.uoff[g] : a.db.eoff[g * a.P];
        const int r1 = MODE == PF_HS ? a.db.uoff[g + 1] : a.db.eoff[(g + 1) * a.P];
        const int nt = (r1 - r0 + BM - 1) / BM;
        if (m < nt) {
            t.g = g;
            t.r0 = r0 + m * BM;
            t.r1 = min(r1, t.r0 + BM);
            return true;
        }
        m -= nt;
    }
    return false;
}

// Per-thread sources, fixed for the whole K range: round i of the activation
// DMA reads row r0 + 32 i + (4 w + l / 16) and round i of the weight DMA column
// 128 i + 16 w + l / 4, so one base pointer per operand and a uniform stride
// give every round.  Activation rows past r1 read the next rows of the buffer
// (the workspace holds BM spare rows past the last one); they only reach
// output rows that are never stored.
struct PfSrc {
    const uint16_t* a;              // round 0's activation row, at this lane's 16-byte segment
    size_t a_step;                  // elements between rounds (32 rows)
    const uint16_t* ag[BM / 32];    // Z1: each round's gathered x row (at the lane's segment)
    const uint8_t* b;               // round 0's weight column, at this lane's 16-byte segment
    size_t b_step;                  // bytes between rounds (128 columns)
    const uint16_t* s;              // scale row of this lane's first column
    size_t sstride;                 // elements between the scale rows of 16 columns
};

// Activation tile: 128 rows x 16 slots; wave w, round i covers rows 32 i + 4 w
// .. + 3 (1 KB, lane-contiguous); lane l writes slot l % 16 of its row and
// fetches the row's global segment (l % 16) ^ (row % 16), so that a fragment
// read (16 rows, one segment) hits 16 distinct bank groups.  Weight tile: 256
// columns x 4 slots of 16 bytes, slot = c ^ ((col / 4) % 4) holding the
// column's bytes [16c, 16c + 16); wave w, round i covers columns 128 i + 16 w
// .. + 15.
EM_DEV void pf_src(PfSrc& p, const uint16_t* A, size_t lda, const uint8_t* Wt, size_t wstride,
                   const uint16_t* srow0, size_t sstride, int r0) {
    const int w = wave_id(), l = lane_id();
    const int rsub = 4 * w + (l >> 4);
    const int seg = (l & 15) ^ (rsub & 15);
    p.a = A + (size_t)(r0 + rsub) * lda + 8 * seg;
    p.a_step = 32 * lda;
    const int col = 16 * w + (l >> 2);
    p.b = Wt + (size_t)col * wstride + 16 * ((l & 3) ^ ((col >> 2) & 3));
    p.b_step = 128 * wstride;
    p.s = srow0;
    p.sstride = sstride;
}

// Step k0's loads: the scales of this lane's NJ columns first, then the weight
// and activation tiles (BN / 128 + 4 DMA instructions per thread).
template <int MODE>
EM_DEV void pf_fetch(uint4* As, uint4* Bs, uint32_t (&sb)[PfCfg<MODE>::NJ], const PfSrc& p, int gq, int k0) {
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < PfCfg<MODE>::NJ; ++j) sb[j] = p.s[(size_t)(16 * j) * p.sstride + k0 / gq];
#pragma unroll
    for (int i = 0; i < PfCfg<MODE>::BN / 128; ++i)
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.b + i * p.b_step + (k0 >> 1)),
                                         (lds_ptr_t)(Bs + (128 * i + 16 * w) * 4), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
        const uint16_t* src = MODE == PF_Z1 ? p.ag[i] + k0 : p.a + i * p.a_step + k0;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(As + (32 * i + 4 * w) * SLOTS), 16, 0, 0);
    }
}

// acc[i][j] += (A rows of subtile i) x (16 x scale_j x dequant(B_j)) over one chunk.
template <int MODE>
EM_DEV void pf_compute(floatx4 (&acc)[NI][PfCfg<MODE>::NJ], const uint4* As, const uint4* Bs,
                       const uint32_t (&sbits)[PfCfg<MODE>::NJ]) {
    constexpr int NJ = PfCfg<MODE>::NJ, WN = PfCfg<MODE>::WN;
    const int l = lane_id(), c = l >> 4, li = l & 15;
    const int wn = wave_id();
    uint4 bq[NJ][4];
    float sc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = WN * wn + 16 * j + li;
        dequant_b(Bs[col * 4 + (c ^ ((col >> 2) & 3))], bq[j]);
        sc[j] = 16.0f * fp16_bits_to_f32((uint16_t)sbits[j]);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = 16 * i + li;
        uint4 af[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) af[s] = As[row * SLOTS + ((4 * c + s) ^ li)];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            floatx4 t = mfma_bf16(af[0], bq[j][0], zero4());
            t = mfma_bf16(af[1], bq[j][1], t);
            t = mfma_bf16(af[2], bq[j][2], t);
            t = mfma_bf16(af[3], bq[j][3], t);
            acc[i][j] = fma4(sc[j], t, acc[i][j]);
        }
    }
}

}  // namespace

// One K step in buffer set X of 3: compute step k (in X) while step k + 2 loads
// into X's predecessor, then wait until only step k + 2's loads are in flight.
#define PF_STEP(X, XN, K0)                                                        \
    if ((K0) + 2 * BK < K) {                                                      \
        pf_fetch<MODE>(As##XN, Bs##XN, s##XN, src, gq, (K0) + 2 * BK);            \
        pf_compute<MODE>(acc, As##X, Bs##X, s##X);                                \
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(Cfg::STEP_VM));                     \
    } else {                                                                      \
        pf_compute<MODE>(acc, As##X, Bs##X, s##X);                                \
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                \
    }                                                                             \
    __syncthreads();                                                              \
    if ((K0) + BK >= K) break;

template <int MODE>
__global__ void __launch_bounds__(PF_TH)
pf_gemm(LayerArgs a) {
    using Cfg = PfCfg<MODE>;
    constexpr int BN = Cfg::BN, WN = Cfg::WN, NJ = Cfg::NJ;
    constexpr bool Z = Cfg::Z;
    __shared__ uint4 As0[BM * SLOTS];
    __shared__ uint4 As1[BM * SLOTS];
    __shared__ uint4 As2[BM * SLOTS];
    __shared__ uint4 Bs0[BN * 4];
    __shared__ uint4 Bs1[BN * 4];
    __shared__ uint4 Bs2[BN * 4];
    const int ntn = Z ? 1 : (MODE == PF_HS ? a.h : a.d) / BN;
    // XCD-aware order: XCD x = blockIdx % 8 takes tiles [x * per, (x + 1) * per)
    const int per = gridDim.x >> 3;
    const int b = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    PfTile t;
    if (!pf_tile<MODE>(a, b, ntn, t)) return;

    const int K = (MODE == PF_HS || MODE == PF_Z1) ? a.d : a.h;
    const int N = Z ? a.r : (MODE == PF_HS ? a.h : a.d);
    const int gq = min(a.gq, K);
    const uint16_t* A = MODE == PF_HS ? a.xg : a.act;
    const uint8_t* W = MODE == PF_HS ? a.s_up : (MODE == PF_OUT ? a.s_dn : (MODE == PF_Z1 ? a.a_up : a.a_dn));
    const uint16_t* S = MODE == PF_HS ? a.s_up_s : (MODE == PF_OUT ? a.s_dn_s : (MODE == PF_Z1 ? a.a_up_s : a.a_dn_s));
    const int l = lane_id(), wv = wave_id(), c = l >> 4, li = l & 15;
    const int wn = wv;

    PfSrc src;
    pf_src(src, A, (size_t)K, W + ((size_t)t.g * N + t.n0) * (K / 2), (size_t)(K / 2),
           S + ((size_t)t.g * N + t.n0 + WN * wn + li) * (K / gq), (size_t)(K / gq), t.r0);
    if constexpr (MODE == PF_Z1) {
        // x rows of the tile's tokens (rows past r1 repeat the last row)
        const int rsub = 4 * wv + (l >> 4);
        const int seg = (l & 15) ^ (rsub & 15);
#pragma unroll
        for (int i = 0; i < BM / 32; ++i)
            src.ag[i] = a.x + (size_t)a.db.row_tok[min(t.r0 + 32 * i + rsub, t.r1 - 1)] * a.d + 8 * seg;
    }

    floatx4 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();

    // ---- main loop: three buffer sets, loads two steps ahead of the math (K >= 3 BK)
    uint32_t s0[NJ], s1[NJ], s2[NJ];
    pf_fetch<MODE>(As0, Bs0, s0, src, gq, 0);
    pf_fetch<MODE>(As1, Bs1, s1, src, gq, BK);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(Cfg::STEP_VM));
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += 3 * BK) {
        PF_STEP(0, 2, k0)
        PF_STEP(1, 0, k0 + BK)
        PF_STEP(2, 1, k0 + 2 * BK)
    }

    // ---- R1 / R4 inputs: rounded to bf16, no further terms
    if constexpr (Z) {
        uint16_t* out = MODE == PF_Z1 ? a.z1 : a.z2;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = t.r0 + 16 * i + 4 * c + v;
                if (row >= t.r1) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    out[(size_t)row * a.r + WN * wn + 16 * j + li] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
            }
        return;
    }

    // ---- LoRA branch: V[g] (bf16 [N][rL]) x the rounded LoRA input rows (bf16 [rows][rLp])
    const int rLp = (a.rL + 7) & ~7;
    {
        const uint16_t* V = (MODE == PF_HS ? a.lu_v : a.ld_v) + (size_t)t.g * N * a.rL;
        const uint16_t* Z = MODE == PF_HS ? a.zl : a.zl2;
        for (int kb = 0; kb < a.rL; kb += 32) {
            const bool kv = kb + 8 * c < a.rL;
            uint4 bv[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int n = t.n0 + WN * wn + 16 * j + li;
                bv[j] = kv ? ld16(V + (size_t)n * a.rL + kb + 8 * c) : zero_u4();
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int row = min(t.r0 + 16 * i + li, t.r1 - 1);
                const uint4 av = kv ? ld16(Z + (size_t)row * rLp + kb + 8 * c) : zero_u4();
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_bf16(av, bv[j], acc[i][j]);
            }
        }
    }

    // ---- per-expert delta down: B_dn[e] (int4 [d][r]) x R4 rows of expert e
    if constexpr (MODE == PF_OUT) {
        const int gq_r = min(a.gq, a.r);
        const int e_first = a.db.row_exp[t.r0], e_last = a.db.row_exp[t.r1 - 1];
        for (int e = e_first; e <= e_last; ++e) {
            const int p = max(a.db.eoff[e], t.r0) - t.r0;          // tile rows [p, q) are expert e's
            const int q = min(a.db.eoff[e + 1], t.r1) - t.r0;
            if (p >= q) continue;
            for (int k0 = 0; k0 < a.r; k0 += KC) {
                uint4 bq[NJ][4];
                float sc[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const size_t n = (size_t)e * a.d + t.n0 + WN * wn + 16 * j + li;
                    dequant_b(ld16(a.b_dn + n * (a.r / 2) + (k0 >> 1) + 16 * c), bq[j]);
                    sc[j] = 16.0f * fp16_bits_to_f32(a.b_dn_s[n * (a.r / gq_r) + k0 / gq_r]);
                }
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int rl = 16 * i;        // subtile rows [rl, rl + 16)
                    if (rl + 16 <= p || rl >= q) continue;             // wave-uniform
                    const int row = rl + li;
                    const bool mine = row >= p && row < q;
                    const uint16_t* zr = a.z2 + (size_t)(t.r0 + (mine ? row : p)) * a.r + k0 + 32 * c;
                    uint4 af[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) af[s] = mine ? ld16(zr + 8 * s) : zero_u4();
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        floatx4 tt = mfma_bf16(af[0], bq[j][0], zero4());
                        tt = mfma_bf16(af[1], bq[j][1], tt);
                        tt = mfma_bf16(af[2], bq[j][2], tt);
                        tt = mfma_bf16(af[3], bq[j][3], tt);
                        acc[i][j] = fma4(sc[j], tt, acc[i][j]);
                    }
                }
            }
        }
    }

    // ---- store: lane holds rows 16 i + 4 c + v, column 16 j + li of its wave's block
    float* out = MODE == PF_HS ? a.hs : a.o;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = t.r0 + 16 * i + 4 * c + v;
            if (row >= t.r1) continue;
            float* orow = out + (size_t)row * N + t.n0 + WN * wn + li;
#pragma unroll
            for (int j = 0; j < NJ; ++j) orow[16 * j] = acc[i][j][v];
        }
}

// Delta up, sum and activation for large batches (steps a5 and a7, r = 128):
// a[row] = RNbf16(SiLU(Hs[u(row)] + 16 s * (B_up[e] . z1[row]))) for a 64-row
// task of expert e and 256 columns.  The z1 fragments are loaded once and
// serve four 64-column blocks; each block's 64 x 64 fp32 result goes through
// LDS so that Hs is read and a written as whole row segments (256 and 128
// bytes per row) instead of 64- and 32-byte pieces.
__global__ void __launch_bounds__(256)
pf_act(LayerArgs a) {
    __shared__ float ot[64][64 + 4];
    const int b = blockIdx.x;
    const int s_e = [&] {                                // expert of this 64-row tile
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
    const int l = lane_id(), wv = wave_id(), c = l >> 4, li = l & 15;
    const int n0 = blockIdx.y * 256;

    uint4 af[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
        const int r = rbeg + min(16 * ms + li, rows - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) af[ms][s] = ld16(a.z1 + (size_t)r * KC + 32 * c + 8 * s);
    }
    const int tr = threadIdx.x >> 2, tq = threadIdx.x & 3;   // epilogue: row, 16-column quarter
    const int u = tr < rows ? a.db.row_u[rbeg + tr] : 0;
    for (int cb = 0; cb < 4; ++cb) {
        const size_t n = (size_t)s_e * a.h + n0 + 64 * cb + 16 * wv + li;
        const uint4 raw = ld16(a.b_up + n * (KC / 2) + 16 * c);
        const uint32_t sb = a.b_up_s[n];
        floatx4 acc[4];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) acc[ms] = zero4();
        mac_fast<4>(acc, af, raw, sb);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int v = 0; v < 4; ++v) ot[16 * ms + 4 * c + v][16 * wv + li] = acc[ms][v];
        __syncthreads();
        if (tr < rows) {
            const int col = n0 + 64 * cb + 16 * tq;
            const float4* hp = reinterpret_cast<const float4*>(a.hs + (size_t)u * a.h + col);
            uint32_t ob[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 hv = hp[q];
                const float* o = &ot[tr][16 * tq + 4 * q];
                const uint32_t b0 = f32_to_bf16_rne(silu(o[0] + hv.x));
                const uint32_t b1 = f32_to_bf16_rne(silu(o[1] + hv.y));
                const uint32_t b2 = f32_to_bf16_rne(silu(o[2] + hv.z));
                const uint32_t b3 = f32_to_bf16_rne(silu(o[3] + hv.w));
                ob[2 * q] = b0 | (b1 << 16);
                ob[2 * q + 1] = b2 | (b3 << 16);
            }
            uint4* ap = reinterpret_cast<uint4*>(a.act + (size_t)(rbeg + tr) * a.h + col);
            ap[0] = make_uint4(ob[0], ob[1], ob[2], ob[3]);
            ap[1] = make_uint4(ob[4], ob[5], ob[6], ob[7]);
        }
        __syncthreads();
    }
}

hipError_t launch_act(const LayerArgs& a, hipStream_t s) {
    dim3 grid(a.max_etiles, a.h / 256);
    prof_begin(s);
    pf_act<<<grid, 256, 0, s>>>(a);
    prof_end(s, "pf_delta_up_act");
    return hipGetLastError();
}

// xg[u] = x[ut_tok[u]]: the activation rows of every group's distinct tokens,
// contiguous per group, 16 bytes per thread.
__global__ void __launch_bounds__(256)
pf_gather_x(const uint16_t* __restrict__ x, const int32_t* __restrict__ ut_tok, const int32_t* __restrict__ n_u,
            uint16_t* __restrict__ xg, int d, int64_t umax) {
    const int segs = d / 8;
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;
    if (i >= umax * segs) return;
    const int64_t u = i / segs;
    if (u >= *n_u) return;
    const int s = (int)(i % segs);
    reinterpret_cast<uint4*>(xg + u * d)[s] = reinterpret_cast<const uint4*>(x + (size_t)ut_tok[u] * d)[s];
}

bool prefill_gemm_ok(int d, int h, int r, int rL, int gq) {
    constexpr int BN = PfCfg<PF_HS>::BN;
    return gq % KC == 0 && r % KC == 0 && rL % 8 == 0 && rL <= 32 && d % BN == 0 && h % BN == 0 &&
           d >= 3 * BK && h >= 3 * BK;
}

hipError_t launch_prefill_gemm(const LayerArgs& a, int mode, int64_t max_rows, hipStream_t s) {
    if (mode == PF_Z1 || mode == PF_Z2) {
        // >= sum over experts of ceil(rows_e / BM)
        int64_t blocks = max_rows / BM + (a.E < max_rows ? a.E : max_rows) + 1;
        blocks = (blocks + 7) & ~7ll;
        prof_begin(s);
        if (mode == PF_Z1) {
            pf_gemm<PF_Z1><<<(unsigned)blocks, PF_TH, 0, s>>>(a);
            prof_end(s, "pf_z1");
        } else {
            pf_gemm<PF_Z2><<<(unsigned)blocks, PF_TH, 0, s>>>(a);
            prof_end(s, "pf_z2");
        }
        return hipGetLastError();
    }
    const int ntn = (mode == PF_HS ? a.h : a.d) / PfCfg<PF_HS>::BN;
    const int64_t mt = max_rows / BM + a.G + 1;          // >= sum over groups of ceil(rows_g / BM)
    int64_t blocks = mt * ntn;
    blocks = (blocks + 7) & ~7ll;
    prof_begin(s);
    if (mode == PF_HS) {
        pf_gemm<PF_HS><<<(unsigned)blocks, PF_TH, 0, s>>>(a);
        prof_end(s, "pf_shared_up");
    } else {
        pf_gemm<PF_OUT><<<(unsigned)blocks, PF_TH, 0, s>>>(a);
        prof_end(s, "pf_down");
    }
    return hipGetLastError();
}

hipError_t launch_gather_x(const LayerArgs& a, int64_t umax, hipStream_t s) {
    const int64_t n = umax * (a.d / 8);
    prof_begin(s);
    pf_gather_x<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.x, a.db.ut_tok, a.db.uoff + a.G, a.xg, a.d, umax);
    prof_end(s, "pf_gather_x");
    return hipGetLastError();
}

}  // namespace em
