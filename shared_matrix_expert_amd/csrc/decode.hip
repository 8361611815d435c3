// Expert layer for decode and speculative-verify batches (T <= 64 tokens).
//
// Generation reads weights far more than it computes with them (launch post
// "Edge0-145B: Frontier AI Capabilities on Your Own Computer", Why On-Device
// Models Have Stayed Small; Under the Hood, Scheduling paragraph: verifying
// several draft tokens per weight read spreads that cost).  At these batch
// sizes the layer is bound by HBM: every weight byte of the touched groups and
// experts is streamed once, and the work is cut into three launches so that
// the GPU spends its time streaming rather than between kernels:
//
//   dec_up   shared up (once per token and group), R1 / R2 products (split-K
//            partial sums); zeroes the arrival counters of the next two.
//   dec_act  delta up + LoRA up + shared part, SiLU, R3; then the R4 / R5
//            products over the workgroup's columns as partial sums; the last
//            workgroup of an expert adds the partials in a fixed order.
//   dec_down shared down + delta down + LoRA down per group; the last
//            workgroup of each column block forms y in slot order.
//
// No permutation kernel: every workgroup rebuilds the view of the routing it
// needs (an expert's rows, a group's tokens or rows) from topk_idx in LDS.
// Every cross-workgroup sum is taken in a fixed order, so results are
// bitwise reproducible.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "decode_common.h"
#include "mfma_ops.h"
#include "tile_stream.h"
#include "wave_stream.h"

namespace em {

// ------------------------------------------------------------------ kernel 1 -------
// K elements per LDS block for NS activation subtiles
template <int NS> struct KBlock { static constexpr int value = 512 / NS; };

template <int NS, bool LDSP>
__global__ void __launch_bounds__(256)
dec_up(DecodeArgs a) {
    constexpr int KB = KBlock<NS>::value;
    constexpr int LNS = LDSP ? NS : 1;                 // no LDS tiles in the fallback instance
    constexpr int LKB = LDSP ? KB : 128;
    // the LDS streams of the R1 / R2 tasks and the staged x of the wave-streamed
    // shared up share one buffer (a workgroup runs one task)
    constexpr size_t HS_XS = 32768;                    // bytes of x per stage
    constexpr size_t HS_SM = HS_XS + 4 * 2 * WS_TILE * 16;
    constexpr size_t SM = sizeof(StreamLds<LNS, LKB>) > HS_SM ? sizeof(StreamLds<LNS, LKB>) : HS_SM;
    __shared__ RouteView v;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SM];
    StreamLds<LNS, LKB>& L = *reinterpret_cast<StreamLds<LNS, LKB>*>(smem);
    __shared__ int arow_l[16 * NS];
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < a.E; i += blockDim.x) a.cnt_e[i] = 0u;
        for (int i = threadIdx.x; i < a.d / 64; i += blockDim.x) a.cnt_c[i] = 0u;
    }
    rv_load(v, a.idx, a.R);
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    int b = blockIdx.x;
    const int nbh = a.h / 64;
    const int nHS = a.G * (nbh / HS_RB);
    const int nbr = (a.r + 63) / 64;
    const int nZ1 = a.nxmax * a.S1 * nbr;
    const int ks = a.d / a.S1;
    const int gq = min(a.gq, a.d);
    const bool fast = gq >= KC && (ks / KC) % DEPTH == 0 && (a.d / KC) % DEPTH == 0;
    constexpr bool lds = LDSP;                         // workgroup streaming through LDS

    if (b < nHS) {
        // ---- shared up for the distinct tokens of group g, HS_RB blocks of 64 columns
        const int g = b / (nbh / HS_RB), nb0 = (b % (nbh / HS_RB)) * HS_RB;
        const int nrows = rv_group_tokens(v, g, a.T, a.k, a.P);
        if (nrows == 0) return;
        if (LDSP && NS == 1 && a.gq == KC && a.d % 2048 == 0) {
            // Wave-streamed: x rows of the group's tokens staged in LDS, 32 KB
            // per stage (8 rows x 2048 or 16 rows x 1024 elements), then every
            // wave streams its 16 weight rows of each 64-column block with no
            // workgroup barrier until the next stage.
            const int rp = nrows <= 8 ? 8 : 16;
            const int KX = (int)(HS_XS / 2) / rp;
            uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
            ws_u4* T = reinterpret_cast<ws_u4*>(smem + HS_XS) + wv * 2 * WS_TILE;
            WsAct ar;
            const int arw = min(li, rp - 1);
            ar.row[0] = xs + (size_t)arw * KX;
            ar.sw[0] = arw & 15;
            // Row-major weights: tiles rb * 4 + wv of the 128 rows; decode-tiled
            // weights: tiles 2 wv + rb (each wave reads 4 KB contiguous per block)
            const bool tiled = a.s_up_t != nullptr;
            WsSrc src[HS_RB];
            WsSrcT srct[HS_RB];
            floatx4 acc[HS_RB][1];
#pragma unroll
            for (int rb = 0; rb < HS_RB; ++rb) {
                const size_t r0 = (size_t)g * a.h + (nb0 + rb) * 64 + wv * 16;
                ws_src(src[rb], a.s_up + r0 * (a.d / 2), (size_t)(a.d / 2), a.s_up_s + r0 * (a.d / KC),
                       (size_t)(a.d / KC));
                const size_t tg = (size_t)g * (a.h / 128) + nb0 / 2;     // tile group (128 rows)
                ws_src_t(srct[rb], a.s_up_t + tg * 64 * a.d, a.s_up_s + tg * a.d, a.d / KC, 2 * wv + rb);
                acc[rb][0] = zero4();
            }
            constexpr int XU = HS_XS / 16 / 256;          // 16-byte pieces per thread and stage
            const int spr = KX / 8;                        // 16-byte segments per staged row
            for (int ks = 0; ks < a.d; ks += KX) {
                __syncthreads();                           // the previous stage is read
                uint4 xv[XU];
#pragma unroll
                for (int u = 0; u < XU; ++u) {
                    const int q = (int)threadIdx.x + 256 * u, r = q / spr, sg = q % spr;
                    xv[u] = ld16(a.x + (size_t)v.rtok[min(r, nrows - 1)] * a.d + ks + 8 * sg);
                }
#pragma unroll
                for (int u = 0; u < XU; ++u) {
                    const int q = (int)threadIdx.x + 256 * u, r = q / spr, sg = q % spr;
                    *reinterpret_cast<uint4*>(xs + (size_t)r * KX + 8 * ((sg & ~15) | ((sg & 15) ^ (r & 15)))) = xv[u];
                }
                __syncthreads();
                if (tiled) ws_gemm2_t<1>(acc[0], acc[1], srct[0], srct[1], ks, ar, KX);
                else ws_gemm2<1>(acc[0], acc[1], src[0], src[1], ks, T, ar, KX);
            }
#pragma unroll
            for (int rb = 0; rb < HS_RB; ++rb) {
                const int ncol = tiled ? nb0 * 64 + (2 * wv + rb) * 16 + li : (nb0 + rb) * 64 + wv * 16 + li;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = 4 * c + q;
                    if (i < nrows) a.hs[((size_t)v.rtok[i] * a.G + g) * a.h + ncol] = acc[rb][0][q];
                }
            }
        } else if constexpr (lds) {
            if ((int)threadIdx.x < 16 * NS)
                arow_l[threadIdx.x] = v.rtok[(int)threadIdx.x < nrows ? threadIdx.x : 0];
            __syncthreads();
            const size_t r0 = (size_t)g * a.h + nb0 * 64;
            const StreamArgs sa{a.s_up + r0 * (a.d / 2), (size_t)(a.d / 2), a.s_up_s + r0 * (a.d / gq),
                                (size_t)(a.d / gq), 64, gq, a.x, (size_t)a.d};
            stream_gemm_rows<NS, KB>(L, sa, (size_t)64 * (a.d / 2), (size_t)64 * (a.d / gq), HS_RB, arow_l, nrows,
                                     0, a.d, [&](int rb, const floatx4 (&acc)[NS]) {
                const int ncol = (nb0 + rb) * 64 + wv * 16 + li;
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = ms * 16 + 4 * c + q;
                        if (i < nrows) a.hs[((size_t)v.rtok[i] * a.G + g) * a.h + ncol] = acc[ms][q];
                    }
            });
        } else {
            for (int rb = 0; rb < HS_RB; ++rb) {
                const int ncol = (nb0 + rb) * 64 + wv * 16 + li;
                floatx4 acc[NS];
#pragma unroll
                for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
                const int nsub = (nrows + 15) >> 4;
                const uint8_t* wrow = a.s_up + ((size_t)g * a.h + ncol) * (a.d / 2);
                const uint16_t* srow = a.s_up_s + ((size_t)g * a.h + ncol) * (a.d / gq);
                const uint16_t* arow[NS];
                bool av[NS];
#pragma unroll
                for (int ms = 0; ms < NS; ++ms) {
                    const int i = ms * 16 + li;
                    av[ms] = i < nrows;
                    arow[ms] = a.x + (size_t)v.rtok[av[ms] ? i : 0] * a.d;
                }
                if (fast) stream_i4_fast<NS, DEPTH>(acc, wrow, srow, 0, a.d, gq, arow, c);
                else stream_i4<NS, DEPTH>(acc, wrow, srow, true, 0, a.d, a.d, gq, arow, av, nsub, c);
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = ms * 16 + 4 * c + q;
                        if (i < nrows) a.hs[((size_t)v.rtok[i] * a.G + g) * a.h + ncol] = acc[ms][q];
                    }
            }
        }
        return;
    }
    b -= nHS;
    if (b < nZ1) {
        // ---- R1 input: partial sums of A_up[e] x over one K slice
        const int xi = b / (a.S1 * nbr);
        const int rem = b % (a.S1 * nbr);
        const int s = rem / nbr, nb = rem % nbr;
        const int e = rv_distinct_expert(v, a.R, a.E, xi);
        if (e < 0) return;
        const int nrows = rv_expert_rows(v, e, a.T, a.k);
        const int nsub = (nrows + 15) >> 4;
        const int n0 = nb * 64 + wv * 16;
        const int ncol = n0 + li;
        const bool nvalid = ncol < a.r;
        floatx4 acc[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
        if constexpr (lds) {
            if ((int)threadIdx.x < 16 * NS)
                arow_l[threadIdx.x] = v.rtok[(int)threadIdx.x < nrows ? threadIdx.x : 0];
            __syncthreads();
            const size_t r0 = (size_t)e * a.r + nb * 64;
            const StreamArgs sa{a.a_up + r0 * (a.d / 2), (size_t)(a.d / 2), a.a_up_s + r0 * (a.d / gq),
                                (size_t)(a.d / gq), min(64, a.r - nb * 64), gq, a.x, (size_t)a.d};
            stream_gemm<NS, KB>(acc, L, sa, arow_l, nrows, s * ks, (s + 1) * ks);
        } else {
            if (n0 >= a.r) return;
            const uint8_t* wrow = a.a_up + ((size_t)e * a.r + (nvalid ? ncol : 0)) * (a.d / 2);
            const uint16_t* srow = a.a_up_s + ((size_t)e * a.r + (nvalid ? ncol : 0)) * (a.d / gq);
            const uint16_t* arow[NS];
            bool av[NS];
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) {
                const int i = ms * 16 + li;
                av[ms] = i < nrows;
                arow[ms] = a.x + (size_t)v.rtok[av[ms] ? i : 0] * a.d;
            }
            if (fast) stream_i4_fast<NS, DEPTH>(acc, wrow, srow, s * ks, (s + 1) * ks, gq, arow, c);
            else stream_i4<NS, DEPTH>(acc, wrow, srow, nvalid, s * ks, (s + 1) * ks, a.d, gq, arow, av, nsub, c);
        }
        if (!nvalid) return;
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ms * 16 + 4 * c + q;
                if (i < nrows) a.z1p[((size_t)s * a.R + v.rows[i]) * a.r + ncol] = acc[ms][q];
            }
        return;
    }
    b -= nZ1;
    {
        // ---- R2 input: partial sums of U_up[g] x; wave wv takes a quarter of slice s
        const int g = b / a.S1, s = b % a.S1;
        if (g >= a.G) return;
        const int nrows = rv_group_tokens(v, g, a.T, a.k, a.P);
        if (nrows == 0) return;
        const int kb = s * ks + wv * (ks / 4);
        const int nstep = ks / 4 / 32;                 // steps of 32 elements for this wave
        const uint16_t* arow[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
            const int i = ms * 16 + li;
            arow[ms] = a.x + (size_t)v.rtok[i < nrows ? i : 0] * a.d;
        }
        for (int nt = 0; nt * 16 < a.rL; ++nt) {
            const int n = nt * 16 + li;
            const bool nvalid = n < a.rL;
            const uint16_t* urow = a.lu_u + ((size_t)g * a.rL + (nvalid ? n : 0)) * a.d;
            floatx4 acc[NS];
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
            for (int st0 = 0; st0 < nstep; st0 += 4) {
                uint4 bv[4], av4[4][NS];
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int kk = kb + min(st0 + st, nstep - 1) * 32 + 8 * c;
                    bv[st] = ld16(urow + kk);
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms) av4[st][ms] = ld16(arow[ms] + kk);
                }
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    if (st0 + st < nstep)
#pragma unroll
                        for (int ms = 0; ms < NS; ++ms) acc[ms] = mfma_bf16(av4[st][ms], bv[st], acc[ms]);
            }
            if (!nvalid) continue;
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = ms * 16 + 4 * c + q;
                    if (i < nrows)
                        a.zlp[(((size_t)(s * 4 + wv) * a.T + v.rtok[i]) * a.G + g) * a.rLp + n] = acc[ms][q];
                }
        }
    }
}

// ---- shared up and the R1 / R2 inputs from one work list --------------------------
// Batches of at most 16 tokens with the decode-tiled S_up and A_up.  Every
// token's x row is staged in LDS once per workgroup (1, 4, 8 or 16 rows of d,
// the fewest that hold the batch; the MFMA rows past them repeat the last), so any
// wave can take any weight tile.  The work is a list of items: the 16-row tiles
// of S_up of each group with slots (whole K, 32 KB at d = 4096; outputs for
// every token, the next kernel reads only the group's tokens), then the K
// halves of the 16-row tiles of A_up of each distinct expert (outputs kept for
// the expert's slots, one z1 slice per half).  Wave w takes items w, w + W,
// w + 2W, ... (W waves in the grid): the eight waves of a workgroup read the
// eight tiles of one tile group, one contiguous region, and when every group
// has slots each wave streams two S_up tiles and at most one A_up half.  A
// wave streams its items as a sequence of K halves through one register ring
// that runs across item boundaries; the half's source is worked out once per
// half.  The U_up products (bf16, 16 KB per group and eighth of K) go to the
// last waves, which carry fewer tiled items.
constexpr int UPW_WAVES = 8;
constexpr int UPW_THREADS = 64 * UPW_WAVES;
constexpr int UPW_XS = 16 * 4096;          // staged x elements (RP rows x d)

constexpr int UPW_XMAX = 256;              // distinct experts (the slots of a batch of <= 16 tokens)
constexpr int UPW_MAXK = 8;                // work items per wave

struct UpwLds {
    __attribute__((aligned(16))) uint16_t xs[UPW_XS];
    int16_t glist[64];                     // groups with slots, ascending
    int16_t xlist[UPW_XMAX];               // distinct experts, ascending
    int16_t xslot[UPW_XMAX][16];           // slot of each token for each distinct expert, or -1
    int ng, nx;
};

// The route view, the lists of groups with slots and of distinct experts, and
// each distinct expert's slot per token.
EM_DEV void upw_lists(const DecodeArgs& a, RouteView& v, UpwLds& L) {
    rv_load(v, a.idx, a.R);
    rv_count_experts(v, a.R, a.E);                     // v.ebits: selected experts
    // expert and group lists from the bitmap, built by wave 0: lane w expands
    // word w (32 experts) at its prefix offset; lane g tests group g's bits
    const int nwd = (a.E + 31) >> 5;                    // <= 32 words
    if (wave_id() == 0) {
        const int lane = lane_id();
        const uint32_t word = lane < nwd ? v.ebits[lane] : 0u;
        int pre = __popc(word);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(pre, off, 64);
            if (lane >= off) pre += y;
        }
        int pos = pre - __popc(word);
        for (uint32_t b = word; b; b &= b - 1u) L.xlist[pos++] = (int16_t)(lane * 32 + __ffs(b) - 1);
        if (lane == 63) L.nx = pre;
        bool live = false;
        if (lane < a.G) {
            const int e0 = lane * a.P, e1 = e0 + a.P;  // experts [e0, e1) of group lane
            for (int w = e0 >> 5; w <= (e1 - 1) >> 5; ++w) {
                const int lo = max(e0 - 32 * w, 0), hi = min(e1 - 32 * w, 32);
                const uint32_t m = (hi >= 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
                live = live || (v.ebits[w] & m) != 0u;
            }
        }
        const uint64_t gl = __ballot(live);
        if (live) L.glist[__popcll(gl & ((1ull << lane) - 1ull))] = (int16_t)lane;
        if (lane == 0) L.ng = __popcll(gl);
    }
    __syncthreads();
    // slot of token t for distinct expert xi (-1: the token did not choose it):
    // every slot finds its expert's rank in the bitmap
    for (int i = threadIdx.x; i < L.nx * 16; i += blockDim.x) L.xslot[i >> 4][i & 15] = -1;
    __syncthreads();
    for (int sl = threadIdx.x; sl < a.R; sl += blockDim.x) {
        const int e = v.idx[sl], w = e >> 5;
        int xi = __popc(v.ebits[w] & ((1u << (e & 31)) - 1u));
        for (int u = 0; u < w; ++u) xi += __popc(v.ebits[u]);
        L.xslot[xi][sl / a.k] = (int16_t)sl;
    }
    __syncthreads();
}

// One K half of a work item: its tile source, K half and where it ends.
struct UpwHalf {
    WsSrcT src;
    int kh;          // K half (0, 1)
    int item;        // global item index
    bool last;       // the item's last half: store after it
};

template <int RP, int NBH>
EM_DEV void upw_run(const DecodeArgs& a, RouteView& v, UpwLds& L) {
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    // stage x: RP rows (rows past T repeat row T - 1), 16-byte segments of each
    // row XOR-swizzled by row % 16 in groups of 16.  The loads go out before
    // the route view is built, so that their latency overlaps it.
    constexpr int XU = RP * 4096 / 8 / UPW_THREADS;     // 16-byte pieces per thread at d = 4096
    const int spr = a.d / 8;
    uint4 xv[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int i = (int)threadIdx.x + UPW_THREADS * u;
        const int r = min(i / spr, RP - 1), sg = i % spr;
        xv[u] = ld16(a.x + (size_t)min(r, a.T - 1) * a.d + 8 * sg);
    }
    upw_lists(a, v, L);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int i = (int)threadIdx.x + UPW_THREADS * u;
        const int r = i / spr, sg = i % spr;
        if (r < RP)
            *reinterpret_cast<uint4*>(L.xs + (size_t)r * a.d + 8 * ((sg & ~15) | ((sg & 15) ^ (r & 15)))) = xv[u];
    }
    __syncthreads();
    WsAct ar;
    {
        const int r = min(li, RP - 1);
        ar.row[0] = L.xs + (size_t)r * a.d;
        ar.sw[0] = r & 15;
    }
    const int tgh = a.h / 128;                          // S_up tile groups per group
    const int n_hs = L.ng * tgh * 8;                    // S_up tiles (whole K)
    const int n_z1 = L.nx * (a.r / 16) * 2;             // A_up tile halves
    const int n_items = n_hs + n_z1;
    const int nw = (int)gridDim.x * UPW_WAVES;
    // Items go to the waves in turn.  Numbered workgroup by workgroup, a
    // workgroup's eight waves stream one contiguous tile group; but when most
    // waves hold one or two items, the last round then lands on the first
    // CUs only (at one token: twice the bytes on 148 of 256 CUs), so below two
    // items per wave the waves are numbered across the CUs first.
    const int gw = n_items < 2 * nw ? wv * (int)gridDim.x + (int)blockIdx.x : (int)blockIdx.x * UPW_WAVES + wv;
    const int nk_hs = gw < n_hs ? (n_hs - 1 - gw) / nw + 1 : 0;
    const int nk = gw < n_items ? (n_items - 1 - gw) / nw + 1 : 0;
    const int nhalf = 2 * nk_hs + (nk - nk_hs);         // K halves to stream
    // half hk of this wave (clamped to the last one)
    auto half_of = [&](int hk, UpwHalf& u) {
        hk = min(hk, max(nhalf - 1, 0));
        if (hk < 2 * nk_hs) {
            const int i = gw + (hk >> 1) * nw;
            const int t = i & 7, tg = i >> 3;           // tg over (group list, tile group)
            const int gl = tg / tgh, tgl = tg - gl * tgh;
            const size_t tgi = (size_t)L.glist[gl] * tgh + tgl;
            ws_src_t(u.src, a.s_up_t + tgi * 64 * a.d, a.s_up_s + tgi * a.d, a.d / KC, t);
            u.kh = hk & 1;
            u.item = i;
            u.last = (hk & 1) == 1;
        } else {
            const int i = gw + (nk_hs + hk - 2 * nk_hs) * nw;
            const int j = i - n_hs;
            const int t = j & 7, hh = (j >> 3) & 1, x2 = j >> 4;   // x2 over (expert list, tile group of r)
            const int xi = x2 / (a.r / 128), tgr = x2 - xi * (a.r / 128);
            const size_t tgi = (size_t)L.xlist[xi] * (a.r / 128) + tgr;
            ws_src_t(u.src, a.a_up_t + tgi * 64 * a.d, a.a_up_s + tgi * a.d, a.d / KC, t);
            u.kh = hh;
            u.item = i;
            u.last = true;
        }
    };
    // Outputs are stored after the stream: a global store in the loop would
    // leave stores and loads pending on the same counter, which the compiler
    // then treats as completing out of order and answers with full waits.  The
    // last UPW_MAXK items' results stay in registers, oldest first; rows
    // without an output write a scratch word.
    auto store = [&](int i, const floatx4& acc) {
        float* dst[4];
        if (i < n_hs) {
            const int t = i & 7, tg = i >> 3;
            const int gl = tg / tgh, tgl = tg - gl * tgh;
            const int g = L.glist[gl];
            const int col = tgl * 128 + t * 16 + li;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int tok = 4 * c + q;
                dst[q] = tok < a.T ? a.hs + ((size_t)tok * a.G + g) * a.h + col : a.scratch + lane;
            }
        } else {
            const int j = i - n_hs;
            const int t = j & 7, hh = (j >> 3) & 1, x2 = j >> 4;
            const int xi = x2 / (a.r / 128), tgr = x2 - xi * (a.r / 128);
            const int col = tgr * 128 + t * 16 + li;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int slot = L.xslot[xi][4 * c + q];
                dst[q] = slot >= 0 ? a.z1p + ((size_t)hh * a.R + slot) * a.r + col : a.scratch + lane;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) *dst[q] = acc[q];
    };
    static_assert(WS_RING == 4 && NBH % WS_RING == 0, "a K half is a whole number of four-block turns");
    if (nhalf > 0) {
        // ring slot j holds the codes of block j (mod 4) of the wave's sequence
        // of halves; the scale pairs of a turn of four blocks come in one load,
        // one turn ahead
        ws_u4 w0[WS_RING], w1[WS_RING];
        UpwHalf cur, nxt;
        half_of(0, cur);
        half_of(1, nxt);
        // the first turn's scales, then the codes in slot order, as the loop
        // body issues them (the empty asm statements keep the compiler from
        // reordering them): the waits at the loop head hold for the first
        // iteration and every later one alike
        ws_u4 scc = ws_scales4_t(cur.src, cur.kh * NBH);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < WS_RING; ++j) {
            ws_fetch_tq(w0[j], w1[j], cur.src, cur.kh * NBH + j, 2 * NBH);
            asm volatile("" ::: "memory");
        }
        floatx4 acc[1] = {zero4()};
        floatx4 keep[UPW_MAXK];
#pragma unroll
        for (int i = 0; i < UPW_MAXK; ++i) keep[i] = zero4();
        for (int hk = 0; hk < nhalf; ++hk) {
#pragma unroll
            for (int b0 = 0; b0 < NBH; b0 += WS_RING) {
                // the next turn's scales: later in this half, or the next half's first
                const ws_u4 scn = b0 + WS_RING < NBH ? ws_scales4_t(cur.src, cur.kh * NBH + b0 + WS_RING)
                                                     : ws_scales4_t(nxt.src, nxt.kh * NBH);
                asm volatile("" ::: "memory");
#pragma unroll
                for (int j = 0; j < WS_RING; ++j) {
                    const int b = b0 + j;
                    const uint32_t spair = j == 0 ? scc.x : (j == 1 ? scc.y : (j == 2 ? scc.z : scc.w));
                    ws_block_t<1>(acc, w0[j], w1[j], spair, ar, (cur.kh * NBH + b) * WS_KB);
                    // the block four ahead: later in this half, or early in the next
                    if (b + WS_RING < NBH)
                        ws_fetch_tq(w0[j], w1[j], cur.src, cur.kh * NBH + b + WS_RING, 2 * NBH);
                    else
                        ws_fetch_tq(w0[j], w1[j], nxt.src, nxt.kh * NBH + b + WS_RING - NBH, 2 * NBH);
                }
                scc = scn;
            }
            if (cur.last) {
#pragma unroll
                for (int i = 0; i + 1 < UPW_MAXK; ++i) keep[i] = keep[i + 1];
                keep[UPW_MAXK - 1] = acc[0];
                acc[0] = zero4();
            }
            cur = nxt;
            half_of(hk + 2, nxt);
        }
        // item k of the wave sits at keep[UPW_MAXK - nk + k]
#pragma unroll
        for (int i = 0; i < UPW_MAXK; ++i) {
            const int k = i - (UPW_MAXK - nk);
            if (k >= 0) store(gw + k * nw, keep[i]);
        }
    }
    // U_up x for the last waves: item z = (group list index, eighth of K)
    const int n_zl = L.ng * 8;
    const int zi = nw - 1 - gw;
    if (zi < n_zl) {
        const int g = L.glist[zi >> 3], s8 = zi & 7;
        const int kb = s8 * (a.d / 8);
        for (int nt = 0; nt * 16 < a.rL; ++nt) {
            const int n = nt * 16 + li;
            const uint16_t* urow = a.lu_u + ((size_t)g * a.rL + min(n, a.rL - 1)) * a.d + kb + 8 * c;
            floatx4 acc = zero4();
            for (int st0 = 0; st0 < a.d / 8 / 32; st0 += 4) {
                uint4 bv[4];
#pragma unroll
                for (int st = 0; st < 4; ++st) bv[st] = ld16(urow + (st0 + st) * 32);
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    // A fragment: x row li at K kb + (st0 + st) 32 + 8 c (swizzled segment)
                    const int seg = ((kb + (st0 + st) * 32) >> 3) + c;
                    const int sw = ((seg & 15) ^ ar.sw[0]) | (seg & ~15);
                    const uint4 av = *reinterpret_cast<const uint4*>(ar.row[0] + 8 * sw);
                    acc = mfma_bf16(av, bv[st], acc);
                }
            }
            if (n < a.rL) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int tok = 4 * c + q;
                    if (tok < a.T) a.zlp[(((size_t)s8 * a.T + tok) * a.G + g) * a.rLp + n] = acc[q];
                }
            }
        }
    }
}

__global__ void __launch_bounds__(UPW_THREADS)
dec_up_ws(DecodeArgs a) {
    __shared__ RouteView v;
    __shared__ UpwLds L;
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < a.E; i += blockDim.x) a.cnt_e[i] = 0u;
        for (int i = threadIdx.x; i < a.d / 64; i += blockDim.x) a.cnt_c[i] = 0u;
    }
    if (a.d == 4096) {
        if (a.T == 1) upw_run<1, 8>(a, v, L);
        else if (a.T <= 4) upw_run<4, 8>(a, v, L);
        else if (a.T <= 8) upw_run<8, 8>(a, v, L);
        else upw_run<16, 8>(a, v, L);
    } else {
        if (a.T == 1) upw_run<1, 4>(a, v, L);
        else if (a.T <= 4) upw_run<4, 4>(a, v, L);
        else if (a.T <= 8) upw_run<8, 4>(a, v, L);
        else upw_run<16, 4>(a, v, L);
    }
}

// ------------------------------------------------------------------ kernel 2 -------
// LDS row strides (elements) of the staged bf16 operands, padded against bank conflicts.
constexpr int ZS_W = 264;     // z1 rows, r <= 256
constexpr int ZL_W = 40;      // zl rows, rLp <= 32
constexpr int AS_W = 520;     // activation rows of the workgroup's columns, cb2 <= 512

// bf16 operand from LDS: elements [kk, kk+8) of a row, zero beyond K or for an invalid row.
EM_DEV uint4 lds_a(const uint16_t* row, int kk, int K, bool valid) {
    uint4 v = zero_u4();
    if (!valid || kk >= K) return v;
    v = *reinterpret_cast<const uint4*>(row + kk);
    const int n = K - kk;
    if (n < 8) {
        uint32_t* u = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (2 * i >= n) u[i] = 0u;
            else if (2 * i + 1 >= n) u[i] &= 0xFFFFu;
        }
    }
    return v;
}

template <int NS>
__global__ void __launch_bounds__(256)
dec_act_direct(DecodeArgs a) {
    __shared__ RouteView v;
    __shared__ __attribute__((aligned(16))) uint16_t zs[16 * NS][ZS_W];
    __shared__ __attribute__((aligned(16))) uint16_t zls[16 * NS][ZL_W];
    __shared__ __attribute__((aligned(16))) uint16_t as_[16 * NS][AS_W];
    rv_load(v, a.idx, a.R);
    const int xi = blockIdx.x / a.ncb2, cb = blockIdx.x % a.ncb2;
    const int e = rv_distinct_expert(v, a.R, a.E, xi);
    if (e < 0) return;
    const int nrows = rv_expert_rows(v, e, a.T, a.k);
    const int g = e / a.P;
    const int nsub = (nrows + 15) >> 4;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int gq_r = min(a.gq, a.r);
    const int gq_h = min(a.gq, a.h);
    // one chunk, one scale, whole 16-byte rows of V: the branch-free variant
    const bool fast = a.r == KC && gq_r == KC && a.rL % 8 == 0 && gq_h >= KC;

    // ---- R1, R2: finish the split-K sums in slice order and round to bf16
    for (int i = threadIdx.x; i < 16 * NS * ZS_W; i += blockDim.x) {
        const int row = i / ZS_W, col = i % ZS_W;
        if (row >= nrows || col >= a.r) zs[row][col] = 0;
    }
    for (int i = threadIdx.x; i < 16 * NS * ZL_W; i += blockDim.x) {
        const int row = i / ZL_W, col = i % ZL_W;
        if (row >= nrows || col >= a.rL) zls[row][col] = 0;
    }
    for (int i = threadIdx.x; i < nrows * a.r; i += blockDim.x) {
        const int row = i / a.r, col = i % a.r;
        const float sum = ordered_sum(a.z1p + (size_t)v.rows[row] * a.r + col, a.S1, (size_t)a.R * a.r);
        zs[row][col] = (uint16_t)f32_to_bf16_rne(sum);
    }
    for (int i = threadIdx.x; i < nrows * a.rL; i += blockDim.x) {
        const int row = i / a.rL, col = i % a.rL;
        const float sum = ordered_sum(a.zlp + ((size_t)v.rtok[row] * a.G + g) * a.rLp + col, 4 * a.S1,
                                      (size_t)a.T * a.G * a.rLp);
        zls[row][col] = (uint16_t)f32_to_bf16_rne(sum);
    }
    __syncthreads();

    // ---- h = shared + B_up[e] z1 + V_up[g] zl; a = R3(SiLU(h)) for this wave's columns
    const int ncw = a.cb2 / 4;                        // columns per wave: 32, 64 or 128
    const int col0 = cb * a.cb2 + wv * ncw;
    int tq[NS][4];                                    // token of each output row of this lane
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = ms * 16 + 4 * c + q;
            tq[ms][q] = v.rtok[i < nrows ? i : 0];
        }
    for (int nt0 = 0; nt0 < ncw / 16; nt0 += 4) {
        // issue the loads of 4 column tiles before any arithmetic
        uint4 raw[4], vb[4];
        uint32_t sb[4];
        float hv[4][NS][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int nt = min(nt0 + u, ncw / 16 - 1);
            const int ncol = col0 + nt * 16 + li;
            if (fast) {
                raw[u] = ld16(a.b_up + ((size_t)e * a.h + ncol) * (KC / 2) + 16 * c);
                sb[u] = a.b_up_s[(size_t)e * a.h + ncol];
                const uint4 t = ld16(a.lu_v + ((size_t)g * a.h + ncol) * a.rL + min(8 * c, a.rL - 8));
                vb[u] = 8 * c < a.rL ? t : zero_u4();
            }
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[u][ms][q] = a.hs[((size_t)tq[ms][q] * a.G + g) * a.h + ncol];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int nt = nt0 + u;
            if (nt >= ncw / 16) break;
            const int ncol = col0 + nt * 16 + li;
            floatx4 acc[NS];
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
            if (fast) {
                uint4 af[NS][4];
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        af[ms][s] = *reinterpret_cast<const uint4*>(&zs[ms * 16 + li][32 * c + 8 * s]);
                mac_fast<NS>(acc, af, raw[u], sb[u]);
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
                    acc[ms] = mfma_bf16(*reinterpret_cast<const uint4*>(&zls[ms * 16 + li][8 * c]), vb[u], acc[ms]);
            } else {
                const uint8_t* brow = a.b_up + ((size_t)e * a.h + ncol) * (a.r / 2);
                const uint16_t* bsrow = a.b_up_s + ((size_t)e * a.h + ncol) * (a.r / gq_r);
                const uint16_t* vrow = a.lu_v + ((size_t)g * a.h + ncol) * a.rL;
                for (int k0 = 0; k0 < a.r; k0 += KC) {
                    const int kv = min(KC, a.r - k0);
                    const uint4 rw = load_b_i4(brow, k0 + 32 * c, a.r);
                    const uint2 sc2 = load_scales(bsrow, k0, gq_r, kv, true);
                    uint4 af[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            af[ms][s] = lds_a(&zs[ms * 16 + li][0], k0 + 32 * c + 8 * s, a.r, true);
                    mac_i4<NS>(acc, af, nsub, rw, sc2, gq_r, kv, c);
                }
                for (int kb = 0; kb < a.rL; kb += 32) {
                    const uint4 bv = load_b_bf16(vrow, kb + 8 * c, a.rL);
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
                        acc[ms] = mfma_bf16(lds_a(&zls[ms * 16 + li][0], kb + 8 * c, a.rL, true), bv, acc[ms]);
                }
            }
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = ms * 16 + 4 * c + q;
                    uint16_t ab = 0;
                    if (i < nrows) {
                        ab = (uint16_t)f32_to_bf16_rne(silu(acc[ms][q] + hv[u][ms][q]));
                        a.act[(size_t)v.rows[i] * a.h + ncol] = ab;
                    }
                    as_[i][wv * ncw + nt * 16 + li] = ab;
                }
        }
    }
    __syncthreads();

    // ---- R4, R5 inputs: partial sums over this workgroup's columns; columns
    // [0, r16) hold A_dn[e] rows, [r16, r16 + rL) hold U_dn[g] rows
    const int r16 = (a.r + 15) & ~15;
    const int N2 = r16 + ((a.rL + 15) & ~15);
    const int nt2n = N2 / 16;
    for (int nt2 = wv; nt2 < nt2n; nt2 += 4) {
        const int n2 = nt2 * 16 + li;
        floatx4 acc[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
        if (nt2 * 16 < r16) {
            const bool nvalid = n2 < a.r;
            const uint8_t* wrow = a.a_dn + ((size_t)e * a.r + (nvalid ? n2 : 0)) * (a.h / 2);
            const uint16_t* srow = a.a_dn_s + ((size_t)e * a.r + (nvalid ? n2 : 0)) * (a.h / gq_h);
            if (fast && a.cb2 == 4 * KC) {
                uint4 raw[4];
                uint32_t sb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int kg = cb * a.cb2 + u * KC;
                    raw[u] = ld16(wrow + ((kg + 32 * c) >> 1));
                    sb[u] = srow[kg / gq_h];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    uint4 af[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            af[ms][s] = *reinterpret_cast<const uint4*>(&as_[ms * 16 + li][u * KC + 32 * c + 8 * s]);
                    mac_fast<NS>(acc, af, raw[u], sb[u]);
                }
            } else {
                for (int kk = 0; kk < a.cb2; kk += KC) {
                    const int kg = cb * a.cb2 + kk;
                    const uint4 rw = nvalid ? load_b_i4(wrow, kg + 32 * c, a.h) : zero_u4();
                    const uint2 sb2 = load_scales(srow, kg, gq_h, KC, nvalid);
                    uint4 af[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            af[ms][s] = lds_a(&as_[ms * 16 + li][0], kk + 32 * c + 8 * s, a.cb2, true);
                    mac_i4<NS>(acc, af, nsub, rw, sb2, gq_h, KC, c);
                }
            }
        } else {
            const int cl = n2 - r16;
            const bool nvalid = cl < a.rL;
            const uint16_t* urow = a.ld_u + ((size_t)g * a.rL + (nvalid ? cl : 0)) * a.h + cb * a.cb2;
            for (int kk0 = 0; kk0 < a.cb2; kk0 += 128) {
                uint4 bv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) bv[u] = ld16(urow + kk0 + 32 * u + 8 * c);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (!nvalid) bv[u] = zero_u4();
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
                        acc[ms] = mfma_bf16(*reinterpret_cast<const uint4*>(&as_[ms * 16 + li][kk0 + 32 * u + 8 * c]),
                                            bv[u], acc[ms]);
                }
            }
        }
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ms * 16 + 4 * c + q;
                if (i < nrows) st_agent(&a.z2p[((size_t)cb * a.R + v.rows[i]) * N2 + n2], acc[ms][q]);
            }
    }

    // ---- the last column block of expert e adds the partials in block order
    if (!arrive_last(v, &a.cnt_e[e], (uint32_t)a.ncb2)) return;
    for (int i = threadIdx.x; i < nrows * N2; i += blockDim.x) {
        const int row = i / N2, n2 = i % N2;
        const int slot = v.rows[row];
        const float sum = ordered_sum_agent(a.z2p + (size_t)slot * N2 + n2, a.ncb2, (size_t)a.R * N2);
        const uint16_t bits = (uint16_t)f32_to_bf16_rne(sum);
        if (n2 < a.r) a.z2[(size_t)slot * a.r + n2] = bits;
        else if (n2 >= r16 && n2 - r16 < a.rL) a.zl2[(size_t)slot * a.rLp + (n2 - r16)] = bits;
    }
}

// Activation kernel with every weight block staged through LDS (r = 128,
// quant groups a multiple of 128).  The work is (distinct expert, block of 256
// columns); a fixed grid of workgroups (all resident at once) cuts each
// expert's blocks into the same number of near-equal ranges (as many as the
// grid holds for every expert), so that no range spans two experts and each
// pays the expert's set-up once.  Per block the expert's B_up rows of those columns (256 x 64
// B, contiguous), its A_dn columns (128 rows x 128 B) and the group's U_dn
// columns are loaded coalesced, each phase's next-block loads issued before
// the other phase's arithmetic.  A range keeps its R4 / R5 partial sums in
// registers and stores them once; the expert's last range to arrive adds them
// in block order.
constexpr int CB_L = 256;
constexpr int ACT_RL = 16;        // LoRA rank bound of this kernel (its U_dn block)

// One 256-column block's operands: the B_up share (phase 1) and the A_dn and
// U_dn shares (phase 2), fetched separately so that each is in flight while
// the other phase computes.
struct ActUp {
    uint4 rb[4];
    uint32_t bs;
};
constexpr int ACT_UI = ACT_RL * 32 / 256;   // U_dn 16-byte pieces per thread

struct ActDn {
    uint4 ra[4], ru[ACT_UI];
    uint32_t as2;
};

EM_DEV void act_fetch_up(ActUp& r, const DecodeArgs& a, int e, int cb) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.rb[i] = ld16(a.b_up + ((size_t)e * a.h + cb * CB_L) * (KC / 2) + 16 * (tid + 256 * i));
    r.bs = a.b_up_s[(size_t)e * a.h + cb * CB_L + tid];
}

EM_DEV void act_fetch_dn(ActDn& r, const DecodeArgs& a, int e, int g, int cb) {
    const int tid = threadIdx.x;
    const int gq_h = min(a.gq, a.h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i;
        const int row = q >> 3, seg = q & 7;
        r.ra[i] = ld16(a.a_dn + ((size_t)e * KC + row) * (a.h / 2) + cb * (CB_L / 2) + 16 * seg);
    }
#pragma unroll
    for (int i = 0; i < ACT_UI; ++i) {
        const int q = tid + 256 * i;
        const int urow = q >> 5, useg = q & 31;
        r.ru[i] = ld16(a.ld_u + ((size_t)g * a.rL + min(urow, a.rL - 1)) * a.h + cb * CB_L + 8 * useg);
    }
    r.as2 = a.a_dn_s[((size_t)e * KC + (tid >> 1)) * (a.h / gq_h) + (cb * CB_L + KC * (tid & 1)) / gq_h];
}

template <int NS>
__global__ void __launch_bounds__(256, NS == 1 ? 2 : 1)
dec_act(DecodeArgs a) {
    __shared__ RouteView v;
    __shared__ __attribute__((aligned(16))) uint16_t zs[16 * NS][KC + 8];
    __shared__ __attribute__((aligned(16))) uint16_t zls[16 * NS][ZL_W];
    __shared__ __attribute__((aligned(16))) uint16_t as_[16 * NS][CB_L + 8];
    __shared__ uint4 wb[CB_L * 5];           // B_up block [256][5], then A_dn block [128][9]
    __shared__ uint4 ub[ACT_RL * 33];        // U_dn block [rL][33]
    __shared__ uint16_t bsc[CB_L];
    __shared__ uint16_t asc[KC][2];
    rv_load(v, a.idx, a.R);
    // Work items are (distinct expert, 256-column block), expert-major; each
    // workgroup takes one contiguous range of them (at most a few experts).
    const int X = rv_count_experts(v, a.R, a.E);
    const int NB = a.ncb2;
    const int G0 = (int)gridDim.x;
    const int rpe = max(1, min(NB, G0 / X));          // ranges per expert
    const int tid = threadIdx.x;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int N2 = KC + ((a.rL + 15) & ~15);
    for (int w = blockIdx.x; w < X * rpe; w += G0) {
        // range r of expert xi: blocks [r NB / rpe, (r + 1) NB / rpe)
        const int xi = w / rpe, r = w % rpe;
        const int j0 = (r * NB) / rpe, j1 = ((r + 1) * NB) / rpe;
        const int e = rv_nth_expert(v, a.E, xi);
        const int nrows = rv_expert_rows(v, e, a.T, a.k);
        const int g = e / a.P;

        int tq[NS][4];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ms * 16 + 4 * c + q;
                tq[ms][q] = v.rtok[i < nrows ? i : 0];
            }
        // per-block shared-up values and V_up rows, loaded one block ahead
        uint4 vb[4];
        float hv[4][NS][4];
        auto fetch_hv = [&](int cb, int nt) {
            const int ncol = cb * CB_L + wv * 64 + nt * 16 + li;
            // lanes past the rank re-read the last 8 (finite weights that meet
            // zeros: zl columns past the rank are zero in LDS)
            vb[nt] = ld16(a.lu_v + ((size_t)g * a.h + ncol) * a.rL + min(8 * c, a.rL - 8));
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[nt][ms][q] = a.hs[((size_t)tq[ms][q] * a.G + g) * a.h + ncol];
        };

        // ---- R1, R2: finish the split-K sums in slice order and round to bf16.
        // Every partial is loaded before the first is added (S1 <= 2 slices for
        // R1, 4 S1 <= 8 for R2; addresses past the count are clamped, unused).
        constexpr int ZI = 16 * NS * KC / 256;
        constexpr int ZLI = 16 * NS * 32 / 256;
        float zp[ZI][2], lp[ZLI][8];
        const int s1b = min(1, a.S1 - 1), nl = 4 * a.S1;
#pragma unroll
        for (int u = 0; u < ZI; ++u) {
            const int i = tid + 256 * u, row = min(i / KC, nrows - 1), col = i % KC;
            const float* p = a.z1p + (size_t)v.rows[row] * KC + col;
            zp[u][0] = p[0];
            zp[u][1] = p[(size_t)s1b * a.R * KC];
        }
#pragma unroll
        for (int u = 0; u < ZLI; ++u) {
            const int i = tid + 256 * u, row = min(i / 32, nrows - 1), col = min(i % 32, a.rL - 1);
            const float* p = a.zlp + ((size_t)v.rtok[row] * a.G + g) * a.rLp + col;
#pragma unroll
            for (int s = 0; s < 8; ++s) lp[u][s] = p[(size_t)min(s, nl - 1) * a.T * a.G * a.rLp];
        }
        // then the first block's operands, so that the sums above wait for no
        // weight, in the order the loop issues them (its waits hold for the
        // first pass too only then)
        ActUp ru_;
        ActDn rd_;
        act_fetch_up(ru_, a, e, j0);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) fetch_hv(j0, nt);
        asm volatile("" ::: "memory");
        act_fetch_dn(rd_, a, e, g, j0);
#pragma unroll
        for (int u = 0; u < ZI; ++u) {
            const int i = tid + 256 * u, row = i / KC, col = i % KC;
            float sum = 0.f + zp[u][0];
            if (a.S1 > 1) sum += zp[u][1];
            // one subtile: each 8-element group in the K order (0,4,1,5,2,6,3,7)
            // of dq_offset, so that B_up's codes need no reordering
            const int pcol = NS == 1 ? (col & ~7) | ((col & 3) << 1) | ((col >> 2) & 1) : col;
            zs[row][pcol] = row < nrows ? (uint16_t)f32_to_bf16_rne(sum) : (uint16_t)0;
        }
#pragma unroll
        for (int u = 0; u < ZLI; ++u) {
            const int i = tid + 256 * u, row = i / 32, col = i % 32;
            float sum = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < nl) sum += lp[u][s];
            zls[row][col] = (row < nrows && col < a.rL) ? (uint16_t)f32_to_bf16_rne(sum) : (uint16_t)0;
        }

        floatx4 z2acc[3][NS];                                 // this wave's R4 / R5 tiles nt2 = wv + 4 t
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) z2acc[t][ms] = zero4();
        for (int cb = j0; cb < j1; ++cb) {
            // this block's B_up into LDS; the next block's B_up loads go out at once
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + 256 * i;
                wb[(q >> 2) * 5 + (q & 3)] = ru_.rb[i];
            }
            bsc[tid] = (uint16_t)ru_.bs;
            __syncthreads();
            // unconditional (the last block re-reads itself): the compiler's waits
            // for later loads would otherwise count these as possibly absent
            act_fetch_up(ru_, a, e, min(cb + 1, j1 - 1));

            // ---- h = shared + B_up[e] z1 + V_up[g] zl; a = R3(SiLU(h)).  With
            // one subtile the wave's four column tiles take each K step
            // together, so that their conversions and MFMA chains interleave
            // (the four-subtile instance lacks the registers and keeps one tile
            // at a time).
            if constexpr (NS == 1) {
                uint4 af[NS][4];
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        af[ms][s] = *reinterpret_cast<const uint4*>(&zs[ms * 16 + li][32 * c + 8 * s]);
                // B_up's codes enter the products as 136 + q (dq_offset, with
                // z1 staged in its K order), so each product starts from -136
                // times its z1 row's sum: K = r = 128 is a single quant group,
                // so one such product per row serves every column
                floatx4 zcorr = zero4();
                {
                    const uint4 neg136 = make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u);
#pragma unroll
                    for (int s = 0; s < 4; ++s) zcorr = mfma_bf16(af[0][s], neg136, zcorr);
                }
                uint4 raw[4];
                float sc[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int lrow = wv * 64 + nt * 16 + li;
                    raw[nt] = wb[lrow * 5 + c];
                    sc[nt] = fp16_bits_to_f32(bsc[lrow]);
                }
                floatx4 acc[4][NS];
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const uint32_t w = s == 0 ? raw[nt].x : s == 1 ? raw[nt].y : s == 2 ? raw[nt].z : raw[nt].w;
                        const uint4 b = dq_offset(w);
#pragma unroll
                        for (int ms = 0; ms < NS; ++ms) acc[nt][ms] = mfma_bf16(af[ms][s], b, s == 0 ? zcorr : acc[nt][ms]);
                    }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms) {
                        acc[nt][ms] = fma4(sc[nt], acc[nt][ms], zero4());
                        acc[nt][ms] = mfma_bf16(*reinterpret_cast<const uint4*>(&zls[ms * 16 + li][8 * c]), vb[nt],
                                                acc[nt][ms]);
                    }
                // SiLU only for the rows some lane holds (a wave-uniform test);
                // rows past the expert's count store zeros
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = ms * 16 + 4 * c + q;
                        if (ms * 16 + q < nrows) {
#pragma unroll
                            for (int nt = 0; nt < 4; ++nt) {
                                const uint16_t ab = (uint16_t)f32_to_bf16_rne(silu(acc[nt][ms][q] + hv[nt][ms][q]));
                                as_[i][wv * 64 + nt * 16 + li] = i < nrows ? ab : (uint16_t)0;
                            }
                        } else {
#pragma unroll
                            for (int nt = 0; nt < 4; ++nt) as_[i][wv * 64 + nt * 16 + li] = 0;
                        }
                    }
            } else {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int lrow = wv * 64 + nt * 16 + li;
                    const int ncol = cb * CB_L + lrow;
                    floatx4 acc[NS];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
                    uint4 af[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            af[ms][s] = *reinterpret_cast<const uint4*>(&zs[ms * 16 + li][32 * c + 8 * s]);
                    mac_fast<NS>(acc, af, wb[lrow * 5 + c], bsc[lrow]);
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
                        acc[ms] = mfma_bf16(*reinterpret_cast<const uint4*>(&zls[ms * 16 + li][8 * c]), vb[nt], acc[ms]);
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int i = ms * 16 + 4 * c + q;
                            uint16_t ab = 0;
                            if (i < nrows) ab = (uint16_t)f32_to_bf16_rne(silu(acc[ms][q] + hv[nt][ms][q]));
                            as_[i][lrow] = ab;
                        }
                }
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) fetch_hv(min(cb + 1, j1 - 1), nt);
            __syncthreads();
            // the block's activation rows, 8 bytes per lane, by stores the
            // waits for the operand loads in flight do not count
#pragma unroll
            for (int u = 0; u < 4 * NS; ++u) {
                const int q = tid + 256 * u, row = q >> 6, seg = q & 63;
                if (row < nrows)
                    st8_uncounted(a.act + (size_t)v.rows[row] * a.h + cb * CB_L + 4 * seg,
                                  *reinterpret_cast<const uint64_t*>(&as_[row][4 * seg]));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + 256 * i;
                wb[(q >> 3) * 9 + (q & 7)] = rd_.ra[i];
            }
#pragma unroll
            for (int i = 0; i < ACT_UI; ++i) {
                const int q = tid + 256 * i;
                if ((q >> 5) < a.rL) ub[(q >> 5) * 33 + (q & 31)] = rd_.ru[i];
            }
            asc[tid >> 1][tid & 1] = (uint16_t)rd_.as2;
            __syncthreads();
            act_fetch_dn(rd_, a, e, g, min(cb + 1, j1 - 1));

            // ---- R4, R5 inputs over these 256 columns: 8 tiles of A_dn rows, 1-2 of U_dn rows.
            // With one subtile the wave's two A_dn tiles (wv and wv + 4) take
            // each K step together.
            if constexpr (NS == 1) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    uint4 af[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            af[ms][s] = *reinterpret_cast<const uint4*>(&as_[ms * 16 + li][u * KC + 32 * c + 8 * s]);
                    // A_dn's codes enter as 136 + q in natural K order
                    // (dq_offset_nat); each chunk's products start from -136
                    // times the chunk's activation row sums
                    floatx4 acorr = zero4();
                    {
                        const uint4 neg136 = make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u);
#pragma unroll
                        for (int s = 0; s < 4; ++s) acorr = mfma_bf16(af[0][s], neg136, acorr);
                    }
                    uint4 raw[2];
                    float sc[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int n2 = (wv + 4 * t) * 16 + li;
                        raw[t] = wb[n2 * 9 + u * 4 + c];
                        sc[t] = fp16_bits_to_f32(asc[n2][u]);
                    }
                    floatx4 tp[2][NS];
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const uint32_t w = s == 0 ? raw[t].x : s == 1 ? raw[t].y : s == 2 ? raw[t].z : raw[t].w;
                            const uint4 b = dq_offset_nat(w);
#pragma unroll
                            for (int ms = 0; ms < NS; ++ms) tp[t][ms] = mfma_bf16(af[ms][s], b, s == 0 ? acorr : tp[t][ms]);
                        }
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int ms = 0; ms < NS; ++ms) z2acc[t][ms] = fma4(sc[t], tp[t][ms], z2acc[t][ms]);
                }
                // the U_dn tile (tile wv + 8, past the eight A_dn tiles)
                if (wv + 8 < N2 / 16) {
                    const int cl = (wv + 8) * 16 + li - KC;
                    const bool nvalid = cl < a.rL;
#pragma unroll
                    for (int st = 0; st < CB_L / 32; ++st) {
                        const uint4 bv = nvalid ? ub[cl * 33 + st * 4 + c] : zero_u4();
#pragma unroll
                        for (int ms = 0; ms < NS; ++ms)
                            z2acc[2][ms] = mfma_bf16(*reinterpret_cast<const uint4*>(&as_[ms * 16 + li][st * 32 + 8 * c]),
                                                     bv, z2acc[2][ms]);
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    const int nt2 = wv + 4 * t;
                    if (nt2 >= N2 / 16) break;
                    const int n2 = nt2 * 16 + li;
                    if (nt2 * 16 < KC) {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            uint4 af[NS][4];
#pragma unroll
                            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                                for (int s = 0; s < 4; ++s)
                                    af[ms][s] = *reinterpret_cast<const uint4*>(&as_[ms * 16 + li][u * KC + 32 * c + 8 * s]);
                            mac_fast<NS>(z2acc[t], af, wb[n2 * 9 + u * 4 + c], asc[n2][u]);
                        }
                    } else {
                        const int cl = n2 - KC;
                        const bool nvalid = cl < a.rL;
#pragma unroll
                        for (int st = 0; st < CB_L / 32; ++st) {
                            const uint4 bv = nvalid ? ub[cl * 33 + st * 4 + c] : zero_u4();
#pragma unroll
                            for (int ms = 0; ms < NS; ++ms)
                                z2acc[t][ms] = mfma_bf16(*reinterpret_cast<const uint4*>(&as_[ms * 16 + li][st * 32 + 8 * c]),
                                                         bv, z2acc[t][ms]);
                        }
                    }
                }
            }
            __syncthreads();
        }

        // ---- this range's partial R4 / R5 inputs, stored at the range's first block;
        // the last range of the expert to arrive adds them in block order
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int nt2 = wv + 4 * t;
            if (nt2 >= N2 / 16) break;
            const int n2 = nt2 * 16 + li;
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = ms * 16 + 4 * c + q;
                    if (i < nrows) st_agent(&a.z2p[((size_t)j0 * a.R + v.rows[i]) * N2 + n2], z2acc[t][ms][q]);
                }
        }
        if (arrive_last(v, &a.cnt_e[e], (uint32_t)rpe)) {
            // two outputs per thread, eight ranges' partials of each in flight
            // at once (unconditional loads), added in range order
            constexpr int RU = 8;
            const int n = nrows * N2;
            for (int i0 = tid; i0 < n; i0 += 512) {
                int slot[2], n2v[2];
                float sum[2] = {0.f, 0.f};
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const int i = min(i0 + 256 * it, n - 1), row = i / N2;
                    n2v[it] = i - row * N2;
                    slot[it] = v.rows[row];
                }
                for (int r0 = 0; r0 < rpe; r0 += RU) {
                    int jr[RU];
#pragma unroll
                    for (int u = 0; u < RU; ++u) jr[u] = (min(r0 + u, rpe - 1) * NB) / rpe;
                    float p[2][RU];
#pragma unroll
                    for (int it = 0; it < 2; ++it)
#pragma unroll
                        for (int u = 0; u < RU; ++u)
                            p[it][u] = ld_agent(a.z2p + ((size_t)jr[u] * a.R + slot[it]) * N2 + n2v[it]);
#pragma unroll
                    for (int it = 0; it < 2; ++it)
#pragma unroll
                        for (int u = 0; u < RU; ++u)
                            if (r0 + u < rpe) sum[it] += p[it][u];
                }
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    if (i0 + 256 * it >= n) continue;
                    const uint16_t bits = (uint16_t)f32_to_bf16_rne(sum[it]);
                    const int n2 = n2v[it];
                    if (n2 < KC) a.z2[(size_t)slot[it] * KC + n2] = bits;
                    else if (n2 - KC < a.rL) a.zl2[(size_t)slot[it] * a.rLp + (n2 - KC)] = bits;
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ kernel 3 -------
template <int NS, bool LDSP>
__global__ void __launch_bounds__(256)
dec_down(DecodeArgs a) {
    constexpr int KB = KBlock<NS>::value;
    constexpr int LNS = LDSP ? NS : 1;
    constexpr int LKB = LDSP ? KB : 128;
    __shared__ RouteView v;
    __shared__ StreamLds<LNS, LKB> L;
    __shared__ int arow_l[16 * NS];
    __shared__ int dexp_l[16 * NS];
    __shared__ int dstart_l[16 * NS];
    __shared__ int gcnt[64];
    rv_load(v, a.idx, a.R);
    // rows per group, hence the passes that carry rows: only those workgroups
    // arrive at the column block's counter, so the empty passes of the grid
    // (npass is a bound for the worst routing) never delay the final sum
    if ((int)threadIdx.x < 64) gcnt[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < a.R; i += blockDim.x) atomicAdd(&gcnt[v.idx[i] / a.P], 1);
    __syncthreads();
    int live_passes = 0;
    for (int gg = 0; gg < a.G; ++gg) live_passes += (gcnt[gg] + 16 * NS - 1) / (16 * NS);
    const int nbd = a.d / 64;
    const int pass = blockIdx.x / (a.G * nbd);
    const int g = (blockIdx.x / nbd) % a.G;
    const int nb = blockIdx.x % nbd;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int m0 = pass * 16 * NS;
    int nrows = 0;
    if (rv_group_any(v, g, a.P, a.R)) nrows = rv_group_rows(v, g, a.T, a.k, a.P, a.R);
    const int prow = min(nrows - m0, 16 * NS);          // rows of this pass
    if (prow > 0) {
        const int nsub = (prow + 15) >> 4;
        const int ncol = nb * 64 + wv * 16 + li;
        const int gq = min(a.gq, a.h);
        const int gq_r = min(a.gq, a.r);
        const bool fast = gq >= KC && (a.h / KC) % DEPTH == 0 && a.r == KC && gq_r == KC && a.rL % 8 == 0;
        int slot_i[NS];                                  // slot of the A row this lane supplies
        bool av[NS];
        const uint16_t* arow[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
            const int i = ms * 16 + li;
            av[ms] = i < prow;
            slot_i[ms] = v.rows[m0 + (av[ms] ? i : 0)];
            arow[ms] = a.act + (size_t)slot_i[ms] * a.h;
        }
        // LoRA down operands, issued ahead of the main stream
        const uint16_t* vrow = a.ld_v + ((size_t)g * a.d + ncol) * a.rL;
        uint4 lv = zero_u4(), lz[NS];
        if (fast) {
            const uint4 t = ld16(vrow + min(8 * c, a.rL - 8));
            lv = 8 * c < a.rL ? t : zero_u4();
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) {
                const uint4 z = ld16(a.zl2 + (size_t)slot_i[ms] * a.rLp + min(8 * c, a.rLp - 8));
                lz[ms] = (8 * c < a.rL) ? z : zero_u4();
            }
        }
        floatx4 acc[NS];
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
        const uint8_t* wrow = a.s_dn + ((size_t)g * a.d + ncol) * (a.h / 2);
        const uint16_t* srow = a.s_dn_s + ((size_t)g * a.d + ncol) * (a.h / gq);
        if constexpr (LDSP) {
            if ((int)threadIdx.x < 16 * NS)
                arow_l[threadIdx.x] = v.rows[m0 + ((int)threadIdx.x < prow ? threadIdx.x : 0)];
            __syncthreads();
            const size_t r0 = (size_t)g * a.d + nb * 64;
            const StreamArgs sa{a.s_dn + r0 * (a.h / 2), (size_t)(a.h / 2), a.s_dn_s + r0 * (a.h / gq),
                                (size_t)(a.h / gq), 64, gq, a.act, (size_t)a.h};
            stream_gemm<NS, KB>(acc, L, sa, arow_l, prow, 0, a.h);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) acc[ms] = mfma_bf16(lz[ms], lv, acc[ms]);
        } else if (fast) {
            stream_i4_fast<NS, DEPTH>(acc, wrow, srow, 0, a.h, gq, arow, c);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) acc[ms] = mfma_bf16(lz[ms], lv, acc[ms]);
        } else {
            stream_i4<NS, DEPTH>(acc, wrow, srow, true, 0, a.h, a.h, gq, arow, av, nsub, c);
            for (int kb = 0; kb < a.rL; kb += 32) {
                const uint4 bv = load_b_bf16(vrow, kb + 8 * c, a.rL);
#pragma unroll
                for (int ms = 0; ms < NS; ++ms)
                    if (ms < nsub)
                        acc[ms] = mfma_bf16(load_a(a.zl2 + (size_t)slot_i[ms] * a.rLp, kb + 8 * c, a.rL, av[ms]),
                                            bv, acc[ms]);
            }
        }

        // delta down: one pass per distinct expert among the pass's rows (rows are
        // expert-sorted), the next expert's operands loaded while this one computes
        int my_e = -1, prev_e = -1;
        if (lane < prow) my_e = v.idx[v.rows[m0 + lane]];
        if (lane >= 1 && lane - 1 < prow) prev_e = v.idx[v.rows[m0 + lane - 1]];
        uint64_t starts = __ballot(lane < prow && (lane == 0 || my_e != prev_e));
        if (LDSP && fast) {
            // distinct experts of the pass in row order, and their first rows
            if (wv == 0 && ((starts >> lane) & 1ull)) {
                const int u = __popcll(starts & ((2ull << lane) - 1ull)) - 1;
                dexp_l[u] = my_e;
                dstart_l[u] = lane;
            }
            __syncthreads();
            delta_down_pass<NS>(acc, a, dexp_l, dstart_l, starts, prow, slot_i, ncol);
        } else if (fast) {
            // the A rows (R4 outputs of this pass) are the same for every expert;
            // only the row mask changes.  Each expert needs one 16-byte weight
            // load and one scale, kept DEPTH experts ahead in a ring.
            uint4 af[NS][4];
#pragma unroll
            for (int ms = 0; ms < NS; ++ms)
#pragma unroll
                for (int s = 0; s < 4; ++s) af[ms][s] = ld16(a.z2 + (size_t)slot_i[ms] * KC + 32 * c + 8 * s);
            uint64_t to_fetch = starts, to_do = starts;
            uint4 ring[DEPTH];
            uint32_t sring[DEPTH];
#pragma unroll
            for (int u = 0; u < DEPTH; ++u) {
                const int p = to_fetch ? __ffsll((long long)to_fetch) - 1 : 0;
                to_fetch &= to_fetch - 1;
                const int e = __shfl(my_e, p, kWave);
                const int ee = e < 0 ? 0 : e;
                ring[u] = ld16(a.b_dn + ((size_t)ee * a.d + ncol) * (KC / 2) + 16 * c);
                sring[u] = a.b_dn_s[(size_t)ee * a.d + ncol];
            }
            while (to_do) {
#pragma unroll
                for (int u = 0; u < DEPTH; ++u) {
                    if (!to_do) break;
                    const int p = __ffsll((long long)to_do) - 1;
                    to_do &= to_do - 1;
                    const int pn = to_do ? __ffsll((long long)to_do) - 1 : prow;
                    const uint4 cur = ring[u];
                    const uint32_t scur = sring[u];
                    if (to_fetch) {
                        const int pf = __ffsll((long long)to_fetch) - 1;
                        to_fetch &= to_fetch - 1;
                        const int e = __shfl(my_e, pf, kWave);
                        ring[u] = ld16(a.b_dn + ((size_t)e * a.d + ncol) * (KC / 2) + 16 * c);
                        sring[u] = a.b_dn_s[(size_t)e * a.d + ncol];
                    }
                    // rows [p, pn) belong to this expert: zero the others' A rows
                    uint4 am[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms) {
                        const int i = ms * 16 + li;
                        const bool mine = i >= p && i < pn;
#pragma unroll
                        for (int s = 0; s < 4; ++s) am[ms][s] = mine ? af[ms][s] : zero_u4();
                    }
                    mac_fast<NS>(acc, am, cur, scur);
                }
            }
        } else {
            while (starts) {
                const int p = __ffsll((long long)starts) - 1;
                starts &= starts - 1;
                const int pend = starts ? __ffsll((long long)starts) - 1 : prow;
                const int e = __shfl(my_e, p, kWave);
                const uint8_t* w2 = a.b_dn + ((size_t)e * a.d + ncol) * (a.r / 2);
                const uint16_t* s2 = a.b_dn_s + ((size_t)e * a.d + ncol) * (a.r / gq_r);
                for (int k0 = 0; k0 < a.r; k0 += KC) {
                    const int kv = min(KC, a.r - k0);
                    const uint4 raw2 = load_b_i4(w2, k0 + 32 * c, a.r);
                    const uint2 sb = load_scales(s2, k0, gq_r, kv, true);
                    uint4 af2[NS][4];
#pragma unroll
                    for (int ms = 0; ms < NS; ++ms) {
                        const int i = ms * 16 + li;
                        const bool ok = i >= p && i < pend;
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            af2[ms][s] = ms < nsub ? load_a(a.z2 + (size_t)slot_i[ms] * a.r, k0 + 32 * c + 8 * s, a.r, ok)
                                                   : zero_u4();
                    }
                    mac_i4<NS>(acc, af2, nsub, raw2, sb, gq_r, kv, c);
                }
            }
        }
#pragma unroll
        for (int ms = 0; ms < NS; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ms * 16 + 4 * c + q;
                if (i < prow) st_agent(&a.o[(size_t)v.rows[m0 + i] * a.d + ncol], acc[ms][q]);
            }
    }

    // ---- the last workgroup of this column block forms y = sum_j w_j o_j in slot order
    if (prow <= 0) return;
    if (!arrive_last(v, &a.cnt_c[nb], (uint32_t)live_passes)) return;
    for (int i = threadIdx.x; i < a.T * 64; i += blockDim.x) {
        const int t = i / 64, col = nb * 64 + (i % 64);
        float acc = 0.f;
        for (int j0 = 0; j0 < a.k; j0 += 8) {
            float wv8[8], ov8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = min(j0 + u, a.k - 1);
                wv8[u] = a.topk_w[t * a.k + j];
                ov8[u] = ld_agent(&a.o[(size_t)(t * a.k + j) * a.d + col]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j0 + u < a.k) acc = fmaf(wv8[u], ov8[u], acc);
        }
        a.y[(size_t)t * a.d + col] = acc;
    }
}

// ---- shared down, wave-streamed ----------------------------------------------------
// Batches of at most 16 slots (every group's rows fit one 16-row subtile), r =
// 128, quant groups of 128.  A workgroup of 8 waves takes (group, 128 output
// columns); each wave streams the int4 S_dn rows of its 16 columns (full-line
// loads, four blocks ahead) against the group's activation rows staged
// through LDS in pieces of 1024 elements per row (8 or 16 rows, chosen by the
// row count; a 4-row instance measured slower at verify), then adds the LoRA
// down V_dn zl2 and the delta down of each
// distinct expert.  The per-slot outputs go to the workspace, and the column
// block's last arriving workgroup forms y.  With every group's rows in one
// workgroup, each light group of a decode step fills 32 compute units with
// one full-rate stream.
constexpr int DNW_WAVES = 8;
constexpr int DNW_COLS = 16 * DNW_WAVES;
constexpr int DNW_THREADS = 64 * DNW_WAVES;

struct DnwLds {
    __attribute__((aligned(16))) uint16_t xs[2 * WS_PIECE];   // two staged activation pieces (128 KB)
    ws_u4 tile[DNW_WAVES * WS_TILE];                           // one transposition tile per wave
    int arow[32];                                              // staged row -> slot
    int dexp[32];                                              // distinct experts of the pass, in row order
    int dstart[32];                                            // first row of each
};

// The pass's staged rows (row -> slot) and its distinct experts with their
// first rows: rows are sorted by expert, so an expert starts where the row's
// expert differs from the previous row's.  Returns the bit mask of expert
// starts.
template <int RP>
EM_DEV uint64_t dnw_experts(const RouteView& v, DnwLds& L, int m0, int prow) {
    const int lane = lane_id(), wv = wave_id();
    if ((int)threadIdx.x < RP) L.arow[threadIdx.x] = v.rows[m0 + min((int)threadIdx.x, prow - 1)];
    int my_e = -1, prev_e = -1;
    if (lane < prow) my_e = v.idx[v.rows[m0 + lane]];
    if (lane >= 1 && lane - 1 < prow) prev_e = v.idx[v.rows[m0 + lane - 1]];
    const uint64_t starts = __ballot(lane < prow && (lane == 0 || my_e != prev_e));
    if (wv == 0 && ((starts >> lane) & 1ull)) {
        const int u = __popcll(starts & ((2ull << lane) - 1ull)) - 1;
        L.dexp[u] = my_e;
        L.dstart[u] = lane;
    }
    __syncthreads();
    return starts;
}

template <int RP, bool TILED>
EM_DEV void dnw_pass(const DecodeArgs& a, RouteView& v, DnwLds& L, int g, int nb, int m0, int prow,
                     bool with_delta) {
    constexpr int NS = WsPiece<RP, DNW_THREADS>::NS;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int ncol = nb * DNW_COLS + wv * 16 + li;
    const uint64_t starts = dnw_experts<RP>(v, L, m0, prow);
    int slot_i[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) slot_i[ms] = L.arow[min(ms * 16 + li, RP - 1)];
    // LoRA down operands, in flight during the stream
    const uint16_t* vrow = a.ld_v + ((size_t)g * a.d + ncol) * a.rL;
    const uint4 lvt = ld16(vrow + min(8 * c, a.rL - 8));
    uint4 lzt[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) lzt[ms] = ld16(a.zl2 + (size_t)slot_i[ms] * a.rLp + min(8 * c, a.rLp - 8));

    // shared down
    floatx4 acc[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
    {
        WsPieceSrc<RP, DNW_THREADS> q;
        ws_piece_src<RP, DNW_THREADS>(q, a.act, (size_t)a.h, L.arow);
        if constexpr (TILED) {
            // the workgroup's 128 columns are tile group nb of S_dn[g]
            const size_t tg = (size_t)g * (a.d / 128) + nb;
            WsSrcT src;
            ws_src_t(src, a.s_dn_t + tg * 64 * a.h, a.s_dn_s + tg * a.h, a.h / KC, wv);
            ws_gemm_pieces<RP, DNW_THREADS, NS>(acc, src, a.h, q, L.xs, L.tile + wv * WS_TILE);
        } else {
            WsSrc src;
            const size_t r0 = (size_t)g * a.d + nb * DNW_COLS + wv * 16;
            ws_src(src, a.s_dn + r0 * (a.h / 2), (size_t)(a.h / 2), a.s_dn_s + r0 * (a.h / KC),
                   (size_t)(a.h / KC));
            ws_gemm_pieces<RP, DNW_THREADS, NS>(acc, src, a.h, q, L.xs, L.tile + wv * WS_TILE);
        }
    }
    // LoRA down: K = rL <= 32 in one product
    {
        const uint4 lv = 8 * c < a.rL ? lvt : zero_u4();
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) acc[ms] = mfma_bf16(8 * c < a.rL ? lzt[ms] : zero_u4(), lv, acc[ms]);
    }
    if (with_delta) delta_down_pass<NS>(acc, a, L.dexp, L.dstart, starts, prow, slot_i, ncol);
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int i = ms * 16 + 4 * c + qq;
            if (i < prow) st_agent(&a.o[(size_t)v.rows[m0 + i] * a.d + ncol], acc[ms][qq]);
        }
}

// Share `part` of `nparts` of another group's delta down (the group's rows in
// v, one pass of prow rows): the distinct experts [part E / nparts,
// (part + 1) E / nparts) and their rows, into od.
template <int RP>
EM_DEV void dnw_delta_share(const DecodeArgs& a, RouteView& v, DnwLds& L, int nb, int prow, int part, int nparts) {
    constexpr int NS = WsPiece<RP, DNW_THREADS>::NS;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int ncol = nb * DNW_COLS + wv * 16 + li;
    const uint64_t starts = dnw_experts<RP>(v, L, 0, prow);
    const int nexp = __popcll(starts);
    const int ub = part * nexp / nparts, ue = (part + 1) * nexp / nparts;
    if (ub >= ue) return;
    const int r0 = L.dstart[ub], r1 = ue < nexp ? L.dstart[ue] : prow;
    int slot_i[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) slot_i[ms] = L.arow[min(ms * 16 + li, RP - 1)];
    floatx4 acc[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
    delta_down_pass<NS>(acc, a, L.dexp, L.dstart, starts, prow, slot_i, ncol, ub, ue);
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int i = ms * 16 + 4 * c + qq;
            if (i >= r0 && i < r1) st_agent(&a.od[(size_t)v.rows[i] * a.d + ncol], acc[ms][qq]);
        }
}

// y = sum_j w_j o_j in slot order over one column block; with HANDED, the
// slots set in hot_slots (one bit per slot) add their handed-off delta first
// and store the sum back as the slot's output.
template <bool HANDED>
EM_DEV void dnw_combine(const DecodeArgs& a, int nb, const uint32_t* hot_slots) {
    // two outputs per thread and up to 16 slots each with every load in flight
    // at once (unconditional loads: the compiler's waits stay counted), so the
    // combine is one memory round trip per 1024 outputs
    constexpr int KJ = 16;
    const int n = a.T * DNW_COLS, nt = (int)blockDim.x;
    for (int i0 = threadIdx.x; i0 < n; i0 += 2 * nt) {
        int t[2], col[2];
        float acc[2] = {0.f, 0.f};
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = min(i0 + it * nt, n - 1);
            t[it] = i / DNW_COLS;
            col[it] = nb * DNW_COLS + (i % DNW_COLS);
        }
        for (int j0 = 0; j0 < a.k; j0 += KJ) {
            float wv[2][KJ], ov[2][KJ], dv[2][KJ];
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int u = 0; u < KJ; ++u) {
                    const size_t slot = (size_t)t[it] * a.k + min(j0 + u, a.k - 1);
                    wv[it][u] = a.topk_w[slot];
                    ov[it][u] = ld_agent(&a.o[slot * a.d + col[it]]);
                    if constexpr (HANDED) dv[it][u] = ld_agent(&a.od[slot * a.d + col[it]]);
                }
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int u = 0; u < KJ; ++u) {
                    if (j0 + u >= a.k) break;
                    float o = ov[it][u];
                    if constexpr (HANDED) {
                        const int slot = t[it] * a.k + j0 + u;
                        if ((hot_slots[slot >> 5] >> (slot & 31)) & 1u) {
                            o += dv[it][u];
                            if (i0 + it * nt < n) st_agent(&a.o[(size_t)slot * a.d + col[it]], o);
                        }
                    }
                    acc[it] = fmaf(wv[it][u], o, acc[it]);
                }
        }
#pragma unroll
        for (int it = 0; it < 2; ++it)
            if (i0 + it * nt < n) a.y[(size_t)t[it] * a.d + col[it]] = acc[it];
    }
}

template <bool TILED>
__global__ void __launch_bounds__(DNW_THREADS)
dec_down_ws(DecodeArgs a) {
    __shared__ RouteView v;
    __shared__ DnwLds L;
    __shared__ int gcnt[64];
    const int nbd = a.d / DNW_COLS;
    const int per_pass = a.G * nbd;
    const int pass = blockIdx.x / per_pass;
    const int loc = blockIdx.x % per_pass;
    // a group's column blocks on one XCD (workgroups go to the XCDs in turn),
    // so that its activation rows are read into one L2
    const int bx = per_pass % 8 == 0 ? (loc & 7) * (per_pass / 8) + (loc >> 3) : loc;
    const int g = bx / nbd, nb = bx % nbd;
    rv_load(v, a.idx, a.R);
    if ((int)threadIdx.x < 64) gcnt[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < a.R; i += blockDim.x) atomicAdd(&gcnt[v.idx[i] / a.P], 1);
    __syncthreads();
    // passes that carry rows: only they arrive at the column block's counter
    // group counts one per lane (G <= 64): the plan below is wave-wide
    // arithmetic instead of a loop of LDS reads
    const int lane = lane_id();
    const int gc = lane < a.G ? gcnt[lane] : 0;
    int live_passes = (gc + 31) / 32;                  // passes that carry rows: only they arrive
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) live_passes += __shfl_xor(live_passes, off, kWave);
    const int m0 = pass * 32;
    const int prow = min(gcnt[g] - m0, 32);
    if (prow <= 0) return;
    // Hand-off of the delta down: when every group fits one pass, the groups
    // of more than 16 rows (two subtiles, four times the staged activation of
    // an 8-row group) give their column block's delta to the workgroups of
    // the groups of at most 8 rows, split by distinct experts into equal
    // shares, so that the hot groups' workgroups stop being the critical path.
    // Every workgroup derives the same plan from the group counts.
    const uint64_t hot = __ballot(gc > 16), light = __ballot(gc >= 1 && gc <= 8);
    const bool one_pass = __ballot(gc > 32) == 0ull;
    const int nhot = __popcll(hot), nlight = __popcll(light);
    const int share = (one_pass && nhot > 0) ? nlight / nhot : 0;          // helpers per hot group
    const bool handed = share > 0 && ((hot >> g) & 1ull);
    const int my_light = ((light >> g) & 1ull) ? __popcll(light & ((1ull << g) - 1ull)) : -1;
    int help_g = -1;
    if (share > 0 && my_light >= 0 && my_light < share * nhot) {
        uint64_t hm = hot;
        for (int h = my_light / share; h > 0; --h) hm &= hm - 1ull;         // the (my_light / share)-th hot group
        help_g = __ffsll((long long)hm) - 1;
    }
    rv_group_rows(v, g, a.T, a.k, a.P, a.R);
    if (prow > 24) dnw_pass<32, TILED>(a, v, L, g, nb, m0, prow, !handed);
    else if (prow > 16) dnw_pass<24, TILED>(a, v, L, g, nb, m0, prow, !handed);
    else if (prow > 8) dnw_pass<16, TILED>(a, v, L, g, nb, m0, prow, true);
    else dnw_pass<8, TILED>(a, v, L, g, nb, m0, prow, true);
    if (help_g >= 0) {
        rv_group_rows(v, help_g, a.T, a.k, a.P, a.R);
        dnw_delta_share<32>(a, v, L, nb, gcnt[help_g], my_light % share, share);
    }

    // ---- the last workgroup of this column block forms y = sum_j w_j o_j in
    // slot order (o_j = its stream part + its handed-off delta, stored back)
    if (!arrive_last(v, &a.cnt_c[nb], (uint32_t)live_passes)) return;
    if (share > 0) {
        // the slots of the groups that handed off their delta, one bit each
        __shared__ uint32_t hot_slots[DEC_RMAX / 32];
        for (int i = threadIdx.x; i < (a.R + 31) / 32; i += blockDim.x) hot_slots[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < a.R; i += blockDim.x)
            if (gcnt[v.idx[i] / a.P] > 16) atomicOr(&hot_slots[i >> 5], 1u << (i & 31));
        __syncthreads();
        dnw_combine<true>(a, nb, hot_slots);
    } else {
        dnw_combine<false>(a, nb, nullptr);
    }
}

// ------------------------------------------------------------------ launcher -------
// Workgroups of `kernel` (256 threads) that fit on the current device at once:
// compute units x resident workgroups per unit, cached per kernel and device.
// The cache is written with atomic stores: threads racing on the first call
// compute and store the same value.
template <class K>
static int resident_grid(K kernel) {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, 256, 0) != hipSuccess || per <= 0) per = 1;
        v = cus * per;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}
// Shapes the wave-streamed shared down takes: quant groups of 128, r = 128,
// LoRA rank a multiple of 8 up to 32, h a multiple of one staged piece (1024
// elements) and whole 128-column blocks; row-major weights only for at most 16
// slots (there, the light groups of a decode step; the tiled weights stream
// fast enough for the 32-row passes of larger batches too).
static bool down_ws_ok(const DecodeArgs& a, bool tiled) {
    return (tiled || a.R <= 16) && a.gq == KC && a.r == KC && a.rL % 8 == 0 && a.rL <= 32 && a.rL > 0 && a.h % 1024 == 0 &&
           a.d % DNW_COLS == 0 && a.P <= 64 && a.T <= 64 && a.G <= 64;
}

// Shapes the work-list shared up takes: at most 16 tokens, decode-tiled S_up
// and A_up, quant groups of 128, d = 2048 or 4096 (every token's x row staged
// whole; K halves a whole number of ring turns), r a multiple of 128, two K
// slices of the R1 / R2 partial sums, and at most UPW_MAXK items per wave.
static int device_cus();

static bool up_ws_ok(const DecodeArgs& a) {
    // at most UPW_MAXK items per wave whatever the routing
    const long items = (long)a.G * (a.h / 16) + (long)a.nxmax * (a.r / 16) * 2;
    if (items > (long)UPW_MAXK * device_cus() * UPW_WAVES) return false;
    return a.s_up_t && a.a_up_t && a.T <= 16 && a.R <= UPW_XMAX && a.gq == KC && (a.d == 2048 || a.d == 4096) &&
           a.r % 128 == 0 && a.h % 128 == 0 && a.S1 == 2 && a.rL <= 32 && a.G <= 64;
}

static int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        v = cus;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int NS, bool LDSP>
static hipError_t launch_ns(const DecodeArgs& a, hipStream_t s, int ns_down) {
    const int nbh = a.h / 64, nbr = (a.r + 63) / 64;
    const int g1 = a.G * (nbh / HS_RB) + a.nxmax * a.S1 * nbr + a.G * a.S1;
    const bool upw = LDSP && NS == 1 && up_ws_ok(a);
    prof_begin(s);
    if (upw) {
        dec_up_ws<<<device_cus(), UPW_THREADS, 0, s>>>(a);
        prof_end(s, "dec_up_ws");
    } else {
        dec_up<NS, LDSP><<<g1, 256, 0, s>>>(a);
        prof_end(s, "dec_up");
    }
    prof_begin(s);
    if (LDSP && upw) {
        dec_act<NS><<<resident_grid(dec_act<NS>), 256, 0, s>>>(a);
        prof_end(s, "dec_act");
    } else if (LDSP) {
        dec_act<NS><<<resident_grid(dec_act<NS>), 256, 0, s>>>(a);
        prof_end(s, "dec_act");
    } else {
        dec_act_direct<NS><<<a.nxmax * a.ncb2, 256, 0, s>>>(a);
        prof_end(s, "dec_act_direct");
    }
    prof_begin(s);
    if (LDSP && ns_down == 2 && a.s_dn_t && down_ws_ok(a, true)) {
        dec_down_ws<true><<<a.npass * a.G * (a.d / DNW_COLS), DNW_THREADS, 0, s>>>(a);
        prof_end(s, "dec_down_wst");
    } else if (LDSP && ns_down == 2 && down_ws_ok(a, false)) {
        dec_down_ws<false><<<a.npass * a.G * (a.d / DNW_COLS), DNW_THREADS, 0, s>>>(a);
        prof_end(s, "dec_down_ws");
    } else {
        const int g3 = a.npass * a.G * (a.d / 64);
        if (ns_down == 2) dec_down<2, LDSP><<<g3, 256, 0, s>>>(a);
        else dec_down<4, LDSP><<<g3, 256, 0, s>>>(a);
        prof_end(s, "dec_down");
    }
    return hipGetLastError();
}

int decode_ns_down(int T) { return T <= 16 ? 2 : 4; }

// Batches of 17..64 tokens take the four-subtile kernels.  (A two-subtile
// instance for 17..32 tokens faulted on its first run and is not built.)
static int decode_ns_up(int T) { return T <= 16 ? 1 : 4; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int nsd = decode_ns_down(a.T);
    if (decode_ns_up(a.T) == 1) return a.lds ? launch_ns<1, true>(a, s, nsd) : launch_ns<1, false>(a, s, nsd);
    return a.lds ? launch_ns<4, true>(a, s, nsd) : launch_ns<4, false>(a, s, nsd);
}

// Whether the LDS-streaming kernels apply: quant groups of whole 128-chunks,
// r = 128, whole 16-byte LoRA rows and K ranges that the K-blocks tile.
bool decode_lds_ok(int T, int d, int h, int r, int rL, int gq, int S1) {
    const int ns = decode_ns_up(T);
    const int nsd = decode_ns_down(T);
    return gq % KC == 0 && r == KC && rL % 8 == 0 && rL <= ACT_RL && h % CB_L == 0 &&
           (d / S1) % (512 / ns) == 0 && h % (512 / nsd) == 0;
}

}  // namespace em
