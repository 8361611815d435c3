// Decode and speculative-verify batches (T <= 8) in one persistent launch.
//
// Generation is bound by weight reads, and verifying several draft tokens per
// read spreads that cost (launch post "Edge0-145B: Frontier AI Capabilities on
// Your Own Computer", Why On-Device Models Have Stayed Small; Under the Hood,
// Scheduling paragraph); the layer runs 48 deep (byteiota "Edge0-145B: Run a
// 145B Open-Source Model on Your Laptop", Not Compression - Architecture).  At
// these batch sizes every touched weight byte is streamed once, and the time
// lost between kernels (each launch's ramp and tail) is a large part of a
// step.  Here one workgroup per compute unit pulls tasks from a queue in the
// workspace until it is empty:
//
//   Z1    (expert, K slice)   R1 inputs A_up x, the expert's last slice rounds z1
//   ZL    (group, K slice)    R2 inputs U_up x, the group's last slice rounds zl
//   UP    (group, 128 h cols) S_up x once for every token of the group, plus
//                             V_up zl, plus B_up z1 of each of the group's
//                             experts, SiLU, R3; the R4 / R5 partial sums
//                             A_dn a and U_dn a over these 128 columns
//   Z2    (group, part)       the R4 / R5 sums over the column blocks, rounded
//   DOWN  (group, row pass, 128 d cols, K half)
//                             S_dn a over half of h, then LoRA down and half
//                             of the experts' delta down; the last task of a
//                             column block forms y in slot order
//
// Tasks are taken in this order, and a task only waits for tasks before it,
// which are already held by running workgroups: the queue cannot deadlock
// whatever the grid size, and phases overlap (a group's down tasks start while
// other groups are still in their up tasks).  Every wait is bounded: past the
// bound the workgroup sets an error word and leaves.
//
// Data handed between workgroups (partial sums, rounded low-rank inputs,
// activation rows, expert outputs) is written with device-coherent (sc1)
// stores and read only after its producers have counted their arrival, in
// buffers laid out so that no cache line holds the results of two producers
// that finish at different times.  Counters are read with atomic operations.
#include <atomic>

#include "common.h"
#include "decode_common.h"
#include "kernels.h"
#include "mfma_ops.h"
#include "wave_stream.h"

namespace em {

constexpr int PL_WAVES = 8;
constexpr int PL_THREADS = 64 * PL_WAVES;
constexpr int PL_T = 8;            // tokens (staged x rows)
constexpr int PL_RMAX = 128;       // slots T * k
constexpr int PL_Z1S = 2;          // K slices of A_up x
constexpr int PL_ZLS = 4;          // K slices of U_up x
constexpr int PL_Z2P = 8;          // parts of a group's R4 / R5 reduction
constexpr int PL_ZP = 136;         // LDS row stride (elements) of z1 and activation rows
constexpr uint32_t PL_SPIN_MAX = 1u << 22;

struct PlView {
    int16_t idx[PL_RMAX];          // slot -> expert
    int16_t rows[PL_RMAX];         // row (sorted by expert, then token) -> slot
    int8_t rtok[PL_RMAX];          // row -> token
    int16_t rxi[PL_RMAX];          // row -> distinct-expert index
    int16_t xe[PL_RMAX];           // distinct experts, ascending
    int16_t xoff[PL_RMAX + 1];     // first row of each distinct expert
    int16_t xslot[PL_RMAX][PL_T];  // slot of (distinct expert, token), -1 if none
    int16_t goff[65];              // first row of each group
    int16_t gx[65];                // first distinct expert of each group
    int16_t gl[64];                // groups with rows, most rows first
    int32_t dnpre[65];             // first down task of each listed group
    int X, NG, total, n_z1, n_zl, n_up, n_z2, dn_arrivals;
    int nkh;                       // K parts of a down task (2 when full-K tasks would not fill the GPU)
};

struct PlLds {
    union alignas(16) {
        uint16_t xs[PL_T * 4096];          // staged x rows (d <= 4096)
        uint16_t pieces[2 * WS_PIECE];     // down tasks: two staged activation pieces
    } u;
    alignas(16) uint16_t z1_l[PL_RMAX][PL_ZP];   // the group's z1 rows (up tasks)
    alignas(16) uint16_t a_l[PL_RMAX][PL_ZP];    // the group's activation rows over 128 columns
    float red[PL_WAVES][256];              // per-wave 16 x 16 tiles
    alignas(16) uint16_t zl_l[16][24];     // zl rows of the tokens
    int arow[32], dexp[32], dstart[32];
    int task;
    uint32_t wflag, aflag;
    uint32_t zready;                       // this workgroup has seen every z1 / zl rounded
};

// ------------------------------------------------------------------ helpers -------

EM_DEV void st_agent_u32(void* p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
EM_DEV void st_agent_u64(void* p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
EM_DEV uint64_t ld_agent_u64(const void* p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
EM_DEV uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

EM_DEV uint32_t bf16_pair(float lo, float hi) { return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16); }

// Count one arrival at c once this workgroup's stores have completed.
EM_DEV void pl_publish(uint32_t* c) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// pl_publish that also tells every thread whether this was the last of `expected`.
EM_DEV bool pl_arrive(PlLds& L, uint32_t* c, uint32_t expected) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        L.aflag = old == expected - 1u ? 1u : 0u;
    }
    __syncthreads();
    return L.aflag != 0u;
}

// Wait until *c >= target (thread 0 polls with atomic reads).  False after
// PL_SPIN_MAX polls, with the error word set.
EM_DEV bool pl_wait(PlLds& L, uint32_t* c, uint32_t target, uint32_t* err) {
    if (threadIdx.x == 0) {
        uint32_t ok = 1u, n = 0u;
        // doubling pauses between polls (up to ~0.4 us): waiters do not crowd
        // the counter that producers are adding to
        int pause = 1;
        while (__hip_atomic_fetch_add(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            for (int i = 0; i < pause; ++i) __builtin_amdgcn_s_sleep(1);
            pause = min(2 * pause, 16);
            if (++n > PL_SPIN_MAX) {
                ok = 0u;
                __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        L.wflag = ok;
    }
    __syncthreads();
    return L.wflag != 0u;
}

// ------------------------------------------------------------------ routing view --
// Rows sorted by (expert, token), the distinct experts with their first rows,
// each group's first row and first distinct expert, the groups with rows
// (most rows first) and the task counts.  Every workgroup builds the same view.
EM_DEV void pl_view(const DecodeArgs& a, PlView& V) {
    const int tid = threadIdx.x, R = a.R;
    for (int i = tid; i < R; i += PL_THREADS) V.idx[i] = (int16_t)a.idx[i];
    __syncthreads();
    for (int i = tid; i < R; i += PL_THREADS) {
        const int key = V.idx[i] * 64 + i / a.k;
        int rank = 0;
        for (int j = 0; j < R; ++j) rank += (V.idx[j] * 64 + j / a.k) < key;
        V.rows[rank] = (int16_t)i;
        V.rtok[rank] = (int8_t)(i / a.k);
    }
    __syncthreads();
    if (wave_id() == 0) {
        const int lane = lane_id();
        int base = 0;
        for (int r0 = 0; r0 < R; r0 += 64) {
            const int r = r0 + lane;
            const bool valid = r < R;
            const int e = valid ? V.idx[V.rows[r]] : -1;
            const int pe = (valid && r > 0) ? V.idx[V.rows[r - 1]] : -2;
            const bool st = valid && e != pe;
            const uint64_t m = __ballot(st);
            const int before = __popcll(m & ((1ull << lane) - 1ull));
            if (st) {
                V.xe[base + before] = (int16_t)e;
                V.xoff[base + before] = (int16_t)r;
            }
            if (valid) V.rxi[r] = (int16_t)(base + __popcll(m & ((2ull << lane) - 1ull)) - 1);
            base += __popcll(m);
        }
        if (lane == 0) {
            V.X = base;
            V.xoff[base] = (int16_t)R;
        }
    }
    __syncthreads();
    const int X = V.X;
    for (int i = tid; i < X * PL_T; i += PL_THREADS) V.xslot[i / PL_T][i % PL_T] = -1;
    if (tid <= a.G) {
        const int lim = tid * a.P;
        int nr = 0, nx = 0;
        for (int i = 0; i < R; ++i) nr += V.idx[i] < lim;
        for (int i = 0; i < X; ++i) nx += V.xe[i] < lim;
        V.goff[tid] = (int16_t)nr;
        V.gx[tid] = (int16_t)nx;
    }
    __syncthreads();
    for (int r = tid; r < R; r += PL_THREADS) V.xslot[V.rxi[r]][V.rtok[r]] = V.rows[r];
    if (tid < a.G) {
        const int n = V.goff[tid + 1] - V.goff[tid];
        if (n > 0) {
            int rank = 0;
            for (int g = 0; g < a.G; ++g) {
                const int m = V.goff[g + 1] - V.goff[g];
                rank += m > n || (m == n && g < tid);
            }
            V.gl[rank] = (int16_t)tid;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int ng = 0;
        for (int g = 0; g < a.G; ++g) ng += V.goff[g + 1] > V.goff[g];
        const int nnb = a.d / 128;
        int np = 0;
        for (int i = 0; i < ng; ++i) {
            const int g = V.gl[i];
            np += (V.goff[g + 1] - V.goff[g] + 31) / 32;
        }
        const int nkh = np * nnb < (int)gridDim.x ? 2 : 1;
        V.nkh = nkh;
        int n = 0;
        for (int i = 0; i < ng; ++i) {
            V.dnpre[i] = n;
            const int g = V.gl[i];
            n += (V.goff[g + 1] - V.goff[g] + 31) / 32 * nnb * nkh;
        }
        V.dnpre[ng] = n;
        V.NG = ng;
        V.dn_arrivals = n / nnb;
        V.n_z1 = X * PL_Z1S;
        V.n_zl = ng * PL_ZLS;
        V.n_up = ng * (a.h / 128);
        V.n_z2 = ng * PL_Z2P;
        V.total = V.n_z1 + V.n_zl + V.n_up + V.n_z2 + n;
    }
    __syncthreads();
}

// ------------------------------------------------------------------ Z1 / ZL -------
// A_up x over one K slice for the expert's tokens (all T staged rows go through
// the product; the expert's own are stored), as partial sums; the expert's
// last slice adds them in slice order and rounds z1 (R1).
template <int NBD>
EM_DEV void pl_z1(const DecodeArgs& a, const PlView& V, PlLds& L, const WsAct& ar, int xi, int s) {
    constexpr int NBS = NBD / PL_Z1S;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int e = V.xe[xi];
    WsSrcT src;
    ws_src_t(src, a.a_up_t + (size_t)e * 64 * a.d, a.a_up_s + (size_t)e * a.d, a.d / KC, wv);
    const int b0 = s * NBS;
    ws_u4 w0[NBS], w1[NBS];
    uint32_t sp[NBS];
#pragma unroll
    for (int j = 0; j < NBS; ++j) ws_fetch_t(w0[j], w1[j], sp[j], src, b0 + j, NBD);
    floatx4 acc[1] = {zero4()};
#pragma unroll
    for (int j = 0; j < NBS; ++j) ws_block_t<1>(acc, w0[j], w1[j], sp[j], ar, (b0 + j) * WS_KB);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int tok = 4 * c + q;
        const int slot = tok < a.T ? V.xslot[xi][tok] : -1;
        if (slot >= 0) st_agent(&a.pl_z1p[((size_t)s * a.R + slot) * KC + 16 * wv + li], acc[0][q]);
    }
    if (!pl_arrive(L, &a.pl_ctr[PL_C_Z1E + e], PL_Z1S)) return;
    const int r0 = V.xoff[xi], nr = V.xoff[xi + 1] - r0;
    for (int i = threadIdx.x; i < nr * 64; i += PL_THREADS) {
        const int slot = V.rows[r0 + i / 64], p = i % 64;
        uint64_t t[PL_Z1S];
#pragma unroll
        for (int u = 0; u < PL_Z1S; ++u) t[u] = ld_agent_u64(a.pl_z1p + ((size_t)u * a.R + slot) * KC + 2 * p);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int u = 0; u < PL_Z1S; ++u) {
            s0 += __uint_as_float((uint32_t)t[u]);
            s1 += __uint_as_float((uint32_t)(t[u] >> 32));
        }
        st_agent_u32(a.pl_z1b + (size_t)slot * KC + 2 * p, bf16_pair(s0, s1));
    }
    pl_publish(&a.pl_ctr[PL_C_ZREADY]);
}

// U_up x over one K slice (each wave an eighth of it, summed over the waves in
// order); the group's last slice adds the slices in order and rounds zl (R2).
template <int NBD>
EM_DEV void pl_zl(const DecodeArgs& a, const PlView& V, PlLds& L, const WsAct& ar, int gi, int s) {
    constexpr int KL = NBD * WS_KB / PL_ZLS / PL_WAVES;   // K per wave (64 or 128)
    constexpr int NST = KL / 32;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int g = V.gl[gi];
    const int kb = s * (NBD * WS_KB / PL_ZLS) + wv * KL;
    const uint16_t* urow = a.lu_u + ((size_t)g * a.rL + min(li, a.rL - 1)) * a.d + kb + 8 * c;
    uint4 bv[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) bv[st] = ld16(urow + st * 32);
    floatx4 acc = zero4();
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        const int seg = ((kb + st * 32) >> 3) + c;
        const int sw = ((seg & 15) ^ ar.sw[0]) | (seg & ~15);
        acc = mfma_bf16(lds16(ar.row[0] + 8 * sw), bv[st], acc);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) L.red[wv][(4 * c + q) * 16 + li] = acc[q];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int tok = threadIdx.x / 16, n = threadIdx.x % 16;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < PL_WAVES; ++w) sum += L.red[w][threadIdx.x];
        if (tok < a.T && n < a.rL) st_agent(&a.pl_zlp[(((size_t)s * a.T + tok) * a.G + g) * 16 + n], sum);
    }
    if (!pl_arrive(L, &a.pl_ctr[PL_C_ZLG + g], PL_ZLS)) return;
    if (threadIdx.x < a.T * 8) {
        const int tok = threadIdx.x / 8, p = threadIdx.x % 8, n = 2 * p;
        float s0 = 0.f, s1 = 0.f;
        if (n < a.rL) {
            uint64_t t[PL_ZLS];
#pragma unroll
            for (int u = 0; u < PL_ZLS; ++u)
                t[u] = ld_agent_u64(a.pl_zlp + (((size_t)u * a.T + tok) * a.G + g) * 16 + n);
#pragma unroll
            for (int u = 0; u < PL_ZLS; ++u) {
                s0 += __uint_as_float((uint32_t)t[u]);
                s1 += __uint_as_float((uint32_t)(t[u] >> 32));
            }
        }
        st_agent_u32(a.pl_zlb + ((size_t)tok * a.G + g) * 16 + n, n < a.rL ? bf16_pair(s0, s1) : 0u);
    }
    pl_publish(&a.pl_ctr[PL_C_ZREADY]);
}

// ------------------------------------------------------------------ UP -------------
// One expert's operands over a 128-column block, for this lane: its B_up rows
// (column tiles t = 0..7: row 16 t + lane % 16, K elements [32 c, 32 c + 32)
// of r = 128, c = lane / 16) and its A_dn rows (R4 tiles t: row 16 t + lane %
// 16, the block's columns [32 c, 32 c + 32)), each 8 KB contiguous per wave,
// with one scale per row.
struct PlBlk {
    uint4 bu[8], ad[8];
    uint32_t bs[8], as[8];
};

// One (group, 128-column block).  Every wave streams one 16-row tile of S_up
// (whole K, four blocks ahead) against the staged x rows; the last turn of the
// stream also issues each wave's first expert's B_up rows.  After V_up zl is
// added, the group's distinct experts are dealt to the waves (wave w: experts
// w, w + 8, ...), and a wave takes its expert through the whole block on its
// own: h = S_up x + V_up zl + B_up z1 over the 128 columns for the expert's
// rows, SiLU and R3 into the block's activation rows, then the R4 inputs
// A_dn a over the block as partial sums, with no barrier between the two.  The
// R5 inputs U_dn a of all the group's rows follow one barrier later.
template <int NBD>
EM_DEV bool pl_up(const DecodeArgs& a, const PlView& V, PlLds& L, const WsAct& ar, int gi, int cb) {
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int g = V.gl[gi];
    const int ncb = a.h / 128;
    const int col = cb * 128 + 16 * wv + li;              // this lane's h column in the stream
    const int x0 = V.gx[g], x1 = V.gx[g + 1];
    const int gr0 = V.goff[g], nrg = V.goff[g + 1] - gr0;

    auto fetch_bu = [&](PlBlk& k, int xi) {
        const int e = V.xe[min(xi, x1 - 1)];
        const uint8_t* bu = a.b_up + ((size_t)e * a.h + cb * 128 + li) * (KC / 2) + 16 * c;
#pragma unroll
        for (int t = 0; t < 8; ++t) k.bu[t] = ld16(bu + t * 16 * (KC / 2));
#pragma unroll
        for (int t = 0; t < 8; ++t) k.bs[t] = a.b_up_s[(size_t)e * a.h + cb * 128 + 16 * t + li];
    };
    auto fetch_ad = [&](PlBlk& k, int xi) {
        const int e = V.xe[min(xi, x1 - 1)];
        const uint8_t* ad = a.a_dn_t + ((size_t)e * ncb + cb) * (KC * KC / 2) + li * (KC / 2) + 16 * c;
#pragma unroll
        for (int t = 0; t < 8; ++t) k.ad[t] = ld16(ad + t * 16 * (KC / 2));
#pragma unroll
        for (int t = 0; t < 8; ++t) k.as[t] = a.a_dn_s[((size_t)e * KC + 16 * t + li) * ncb + cb];
    };

    // ---- z1 rows of the group's slots and zl rows of the tokens.  Once this
    // workgroup has seen them all rounded (its earlier up tasks), the loads go
    // out before the stream and land in LDS after it; otherwise they follow
    // the wait after the stream.
    const int tid = threadIdx.x;
    uint4 zv[2], zlv;
    auto z_issue = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + PL_THREADS * u, row = min(i >> 4, nrg - 1);
            zv[u] = ld16(a.pl_z1b + (size_t)V.rows[gr0 + row] * KC + 8 * (i & 15));
        }
        const int tok = min(tid >> 1, a.T - 1);
        zlv = ld16(a.pl_zlb + ((size_t)tok * a.G + g) * 16 + 8 * (tid & 1));
    };
    auto z_store = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + PL_THREADS * u, row = i >> 4;
            if (row < nrg) *reinterpret_cast<uint4*>(&L.z1_l[row][8 * (i & 15)]) = zv[u];
        }
        for (int i = tid + 2 * PL_THREADS; i < nrg * 16; i += PL_THREADS)      // rows past 64
            *reinterpret_cast<uint4*>(&L.z1_l[i >> 4][8 * (i & 15)]) =
                ld16(a.pl_z1b + (size_t)V.rows[gr0 + (i >> 4)] * KC + 8 * (i & 15));
        if (tid < 32) *reinterpret_cast<uint4*>(&L.zl_l[tid >> 1][8 * (tid & 1)]) = (tid >> 1) < a.T ? zlv : zero_u4();
    };
    const bool zr = L.zready != 0u;
    if (zr) z_issue();

    // ---- S_up x (whole K) through a ring of four blocks.  Turns of four blocks
    // run in a loop that refills each slot right after its block (loads in the
    // same order in the prologue and the loop, so the waits count the loads
    // behind them); the last turn refills nothing and instead issues the
    // wave's first expert's B_up rows and the V_up row.
    WsSrcT src;
    const size_t tgi = (size_t)g * ncb + cb;
    ws_src_t(src, a.s_up_t + tgi * 64 * a.d, a.s_up_s + tgi * a.d, a.d / KC, wv);
    ws_u4 w0[WS_RING], w1[WS_RING];
    ws_u4 scc = ws_scales4_t(src, 0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < WS_RING; ++j) {
        ws_fetch_tq(w0[j], w1[j], src, j, NBD);
        asm volatile("" ::: "memory");
    }
    floatx4 acc[1] = {zero4()};
    for (int b0 = 0; b0 < NBD - WS_RING; b0 += WS_RING) {
        const ws_u4 scn = ws_scales4_t(src, b0 + WS_RING);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < WS_RING; ++j) {
            const uint32_t sp = j == 0 ? scc.x : (j == 1 ? scc.y : (j == 2 ? scc.z : scc.w));
            ws_block_t<1>(acc, w0[j], w1[j], sp, ar, (b0 + j) * WS_KB);
            ws_fetch_tq(w0[j], w1[j], src, b0 + WS_RING + j, NBD);
        }
        scc = scn;
    }
    PlBlk bk;
    fetch_bu(bk, x0 + wv);
    uint4 vup = ld16(a.lu_v + ((size_t)g * a.h + col) * a.rL + min(8 * c, a.rL - 8));
#pragma unroll
    for (int j = 0; j < WS_RING; ++j) {
        const uint32_t sp = j == 0 ? scc.x : (j == 1 ? scc.y : (j == 2 ? scc.z : scc.w));
        ws_block_t<1>(acc, w0[j], w1[j], sp, ar, (NBD - WS_RING + j) * WS_KB);
    }
    if (8 * c >= a.rL) vup = zero_u4();

    if (!zr) {
        if (!pl_wait(L, &a.pl_ctr[PL_C_ZREADY], (uint32_t)(V.X + V.NG), &a.pl_ctr[PL_C_ERR])) return false;
        if (tid == 0) L.zready = 1u;
        z_issue();
    }
    fetch_ad(bk, x0 + wv);
    z_store();
    __syncthreads();

    // ---- LoRA up: S_up x + V_up zl per token and column, into LDS (red[t]:
    // column tile t of the block, [token][16 columns])
    {
        const uint4 za = 8 * c < a.rL ? lds16(&L.zl_l[li][8 * c]) : zero_u4();
        acc[0] = mfma_bf16(za, vup, acc[0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) L.red[wv][(4 * c + q) * 16 + li] = acc[0][q];
    }
    // the U_dn rows of the block (R5), in flight during the experts
    uint4 ub[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
        ub[st] = ld16(a.ld_u + ((size_t)g * a.rL + min(li, a.rL - 1)) * a.h + cb * 128 + 32 * st + 8 * c);
    __syncthreads();

    // ---- this wave's experts, each through the whole block
    float* z2p = a.pl_z2p + (size_t)cb * a.R * PL_Z2W;
    for (int xi = x0 + wv; xi < x1; xi += PL_WAVES) {
        const int r0 = V.xoff[xi] - gr0, nr = V.xoff[xi + 1] - V.xoff[xi];
        int tokq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) tokq[q] = V.rtok[gr0 + r0 + min(4 * c + q, nr - 1)];
        {
            uint4 af[1][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) af[0][s] = li < nr ? lds16(&L.z1_l[r0 + li][32 * c + 8 * s]) : zero_u4();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                floatx4 h[1] = {zero4()};
                mac_fast<1>(h, af, bk.bu[t], bk.bs[t]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 4 * c + q;
                    if (row < nr)
                        L.a_l[r0 + row][16 * t + li] =
                            (uint16_t)f32_to_bf16_rne(silu(h[0][q] + L.red[t][tokq[q] * 16 + li]));
                }
            }
        }
        {
            uint4 af[1][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) af[0][s] = li < nr ? lds16(&L.a_l[r0 + li][32 * c + 8 * s]) : zero_u4();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                floatx4 z[1] = {zero4()};
                mac_fast<1>(z, af, bk.ad[t], bk.as[t]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 4 * c + q;
                    if (row < nr) st_agent(&z2p[(size_t)(gr0 + r0 + row) * PL_Z2W + 16 * t + li], z[0][q]);
                }
            }
        }
        if (xi + PL_WAVES < x1) {
            fetch_bu(bk, xi + PL_WAVES);
            fetch_ad(bk, xi + PL_WAVES);
        }
    }
    __syncthreads();

    // ---- the block's activation rows to the workspace (read by the down tasks)
    for (int i = threadIdx.x; i < nrg * 16; i += PL_THREADS) {
        const int row = i >> 4, sg = i & 15;
        const uint4 v = lds16(&L.a_l[row][8 * sg]);
        uint16_t* dst = a.act + (size_t)V.rows[gr0 + row] * a.h + cb * 128 + 8 * sg;
        st_agent_u64(dst, (uint64_t)v.x | ((uint64_t)v.y << 32));
        st_agent_u64(dst + 4, (uint64_t)v.z | ((uint64_t)v.w << 32));
    }
    // ---- R5 inputs over the block: U_dn rows (rL <= 16) against 16-row subtiles of the group's rows
    for (int j = wv; 16 * j < nrg; j += PL_WAVES) {
        floatx4 t = zero4();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 av = 16 * j + li < nrg ? lds16(&L.a_l[16 * j + li][32 * st + 8 * c]) : zero_u4();
            t = mfma_bf16(av, ub[st], t);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int row = 16 * j + 4 * c + qq;
            if (row < nrg && li < a.rL) st_agent(&z2p[(size_t)(gr0 + row) * PL_Z2W + KC + li], t[qq]);
        }
    }
    pl_publish(&a.pl_ctr[PL_C_UP + g]);
    return true;
}

// ------------------------------------------------------------------ Z2 -------------
// Part `part` of a group's R4 / R5 sums: the partials of the h/128 column
// blocks added in block order and rounded to bf16.
EM_DEV bool pl_z2red(const DecodeArgs& a, const PlView& V, PlLds& L, int gi, int part) {
    const int g = V.gl[gi];
    const int ncb = a.h / 128;
    if (!pl_wait(L, &a.pl_ctr[PL_C_UP + g], (uint32_t)ncb, &a.pl_ctr[PL_C_ERR])) return false;
    const int gr0 = V.goff[g], nrg = V.goff[g + 1] - gr0;
    constexpr int NPAIR = (KC + 16) / 2;                 // value pairs per row
    const int nv = nrg * NPAIR;
    const int v0 = part * nv / PL_Z2P, v1 = (part + 1) * nv / PL_Z2P;
    for (int v = v0 + (int)threadIdx.x; v < v1; v += PL_THREADS) {
        const int row = v / NPAIR, p = v % NPAIR;
        const float* base = a.pl_z2p + (size_t)(gr0 + row) * PL_Z2W + 2 * p;
        float s0 = 0.f, s1 = 0.f;
        for (int c0 = 0; c0 < ncb; c0 += 32) {
            uint64_t t[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) t[u] = ld_agent_u64(base + (size_t)min(c0 + u, ncb - 1) * a.R * PL_Z2W);
#pragma unroll
            for (int u = 0; u < 32; ++u)
                if (c0 + u < ncb) {
                    s0 += __uint_as_float((uint32_t)t[u]);
                    s1 += __uint_as_float((uint32_t)(t[u] >> 32));
                }
        }
        const int slot = V.rows[gr0 + row], n2 = 2 * p;
        if (n2 < KC) st_agent_u32(a.z2 + (size_t)slot * KC + n2, bf16_pair(s0, s1));
        else if (n2 - KC < a.rL) st_agent_u32(a.zl2 + (size_t)slot * a.rLp + (n2 - KC), bf16_pair(s0, s1));
    }
    pl_publish(&a.pl_ctr[PL_C_Z2 + g]);
    return true;
}

// ------------------------------------------------------------------ DOWN -----------
// y = sum_j w_j (o_j + od_j) in slot order over one 128-column block (od only
// when the down tasks were split over two K halves).
EM_DEV void pl_combine(const DecodeArgs& a, int nb, int nkh) {
    constexpr int KJ = 16;
    const int n = a.T * 128;
    for (int i = threadIdx.x; i < n; i += PL_THREADS) {
        const int t = i / 128, col = nb * 128 + i % 128;
        float acc = 0.f;
        for (int j0 = 0; j0 < a.k; j0 += KJ) {
            float wv[KJ], ov[KJ], dv[KJ];
#pragma unroll
            for (int u = 0; u < KJ; ++u) {
                const size_t slot = (size_t)t * a.k + min(j0 + u, a.k - 1);
                wv[u] = a.topk_w[slot];
                ov[u] = ld_agent(&a.o[slot * a.d + col]);
                dv[u] = nkh == 2 ? ld_agent(&a.od[slot * a.d + col]) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < KJ; ++u) {
                if (j0 + u >= a.k) break;
                const float o = ov[u] + dv[u];
                if (a.pl_trace_o) a.o[((size_t)t * a.k + j0 + u) * a.d + col] = o;
                acc = fmaf(wv[u], o, acc);
            }
        }
        a.y[(size_t)t * a.d + col] = acc;
    }
}

// One (group, pass of <= 32 rows, 128 output columns, K part kh of nkh): S_dn
// a over the part of h with the rows staged through LDS in pieces, then (first
// part) the LoRA down, and the part's share of the pass's experts' delta down;
// the per-slot result goes to o (first part) or od (second part).
template <int RP>
EM_DEV bool pl_down(const DecodeArgs& a, const PlView& V, PlLds& L, int gi, int pass, int nb, int kh) {
    constexpr int NS = WsPiece<RP, PL_THREADS>::NS;
    const int lane = lane_id(), wv = wave_id(), c = lane >> 4, li = lane & 15;
    const int g = V.gl[gi];
    const int m0 = V.goff[g] + 32 * pass;
    const int prow = min(32, V.goff[g + 1] - m0);
    const int ncol = nb * 128 + 16 * wv + li;
    const int nkh = V.nkh;
    const int hh = a.h / nkh;
    if (!pl_wait(L, &a.pl_ctr[PL_C_UP + g], (uint32_t)(a.h / 128), &a.pl_ctr[PL_C_ERR])) return false;
    // the pass's rows and their distinct experts (rows are sorted by expert)
    if ((int)threadIdx.x < RP) L.arow[threadIdx.x] = V.rows[m0 + min((int)threadIdx.x, prow - 1)];
    int my_e = -1, prev_e = -1;
    if (lane < prow) my_e = V.idx[V.rows[m0 + lane]];
    if (lane >= 1 && lane - 1 < prow) prev_e = V.idx[V.rows[m0 + lane - 1]];
    const uint64_t starts = __ballot(lane < prow && (lane == 0 || my_e != prev_e));
    if (wv == 0 && ((starts >> lane) & 1ull)) {
        const int u = __popcll(starts & ((2ull << lane) - 1ull)) - 1;
        L.dexp[u] = my_e;
        L.dstart[u] = lane;
    }
    __syncthreads();
    int slot_i[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) slot_i[ms] = L.arow[min(ms * 16 + li, RP - 1)];

    floatx4 acc[NS];
#pragma unroll
    for (int ms = 0; ms < NS; ++ms) acc[ms] = zero4();
    {
        WsPieceSrc<RP, PL_THREADS> q;
        ws_piece_src<RP, PL_THREADS>(q, a.act + (size_t)kh * hh, (size_t)a.h, L.arow);
        const size_t tg = (size_t)g * (a.d / 128) + nb;
        WsSrcT src;
        ws_src_t(src, a.s_dn_t + tg * 64 * a.h, a.s_dn_s + tg * a.h, a.h / KC, wv);
        src.w += (size_t)kh * (hh / WS_KB) * 16384;
        src.s += (size_t)kh * (hh / KC);
        ws_gemm_pieces<RP, PL_THREADS, NS>(acc, src, hh, q, L.u.pieces, nullptr);
    }
    // LoRA down and the delta down need the group's rounded R4 / R5 inputs
    if (!pl_wait(L, &a.pl_ctr[PL_C_Z2 + g], (uint32_t)PL_Z2P, &a.pl_ctr[PL_C_ERR])) return false;
    if (kh == 0) {
        const uint4 lv = ld16(a.ld_v + ((size_t)g * a.d + ncol) * a.rL + min(8 * c, a.rL - 8));
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
            const uint4 lz = ld16(a.zl2 + (size_t)slot_i[ms] * a.rLp + min(8 * c, a.rLp - 8));
            acc[ms] = mfma_bf16(8 * c < a.rL ? lz : zero_u4(), 8 * c < a.rL ? lv : zero_u4(), acc[ms]);
        }
    }
    const int nexp = __popcll(starts);
    delta_down_pass<NS>(acc, a, L.dexp, L.dstart, starts, prow, slot_i, ncol, kh * nexp / nkh,
                        (kh + 1) * nexp / nkh);
    float* out = kh ? a.od : a.o;
#pragma unroll
    for (int ms = 0; ms < NS; ++ms)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int i = ms * 16 + 4 * c + qq;
            if (i < prow) st_agent(&out[(size_t)V.rows[m0 + i] * a.d + ncol], acc[ms][qq]);
        }
    if (pl_arrive(L, &a.pl_ctr[PL_C_DN + nb], (uint32_t)V.dn_arrivals)) pl_combine(a, nb, nkh);
    return true;
}

// ------------------------------------------------------------------ kernel ---------
template <int NBD>
__global__ void __launch_bounds__(PL_THREADS, 1)
dec_layer(DecodeArgs a) {
    __shared__ PlView V;
    __shared__ PlLds L;
    const int li = lane_id() & 15;
    // x rows (rows past T repeat row T - 1), 16-byte segments XOR-swizzled by
    // row within groups of 16; the loads go out before the routing view
    constexpr int D = NBD * WS_KB;
    constexpr int XU = PL_T * D / 8 / PL_THREADS;
    constexpr int SPR = D / 8;
    uint4 xv[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int i = (int)threadIdx.x + PL_THREADS * u;
        const int r = i / SPR, sg = i % SPR;
        xv[u] = ld16(a.x + (size_t)min(r, a.T - 1) * D + 8 * sg);
    }
    pl_view(a, V);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int i = (int)threadIdx.x + PL_THREADS * u;
        const int r = i / SPR, sg = i % SPR;
        *reinterpret_cast<uint4*>(L.u.xs + (size_t)r * D + 8 * ((sg & ~15) | ((sg & 15) ^ (r & 15)))) = xv[u];
    }
    if (threadIdx.x == 0) L.zready = 0u;
    __syncthreads();
    WsAct ar;
    ar.row[0] = L.u.xs + (size_t)min(li, PL_T - 1) * D;
    ar.sw[0] = min(li, PL_T - 1) & 15;
    const int ncb = a.h / 128, nnb = a.d / 128;
    auto next_task = [&]() {
        if (threadIdx.x == 0)
            L.task = (int)__hip_atomic_fetch_add(&a.pl_ctr[PL_C_HEAD], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int t = L.task;
        __syncthreads();
        return t;
    };
    // Tasks come in queue order, so once a workgroup draws a down task it
    // never draws another kind: the two loops keep the register demands of
    // the up side and the down side apart.
    const int first_dn = V.n_z1 + V.n_zl + V.n_up + V.n_z2;
    int ti = next_task();
    for (; ti < first_dn; ti = next_task()) {
        int j = ti;
        if (j < V.n_z1) {
            pl_z1<NBD>(a, V, L, ar, j / PL_Z1S, j % PL_Z1S);
            continue;
        }
        j -= V.n_z1;
        if (j < V.n_zl) {
            pl_zl<NBD>(a, V, L, ar, j / PL_ZLS, j % PL_ZLS);
            continue;
        }
        j -= V.n_zl;
        if (j < V.n_up) {
            if (!pl_up<NBD>(a, V, L, ar, j / ncb, j % ncb)) return;
            continue;
        }
        j -= V.n_up;
        if (!pl_z2red(a, V, L, j / PL_Z2P, j % PL_Z2P)) return;
    }
    for (; ti < V.total; ti = next_task()) {
        int j = ti - first_dn;
        int gi = 0;
        while (V.dnpre[gi + 1] <= j) ++gi;
        j -= V.dnpre[gi];
        const int nkh = V.nkh;
        const int pass = j / (nkh * nnb), nb = (j / nkh) % nnb, kh = j % nkh;
        const int g = V.gl[gi];
        const int prow = min(32, V.goff[g + 1] - V.goff[g] - 32 * pass);
        // two staging shapes (8 or 32 rows) keep the kernel within its registers
        const bool ok = prow > 8 ? pl_down<32>(a, V, L, gi, pass, nb, kh) : pl_down<8>(a, V, L, gi, pass, nb, kh);
        if (!ok) return;
    }
}

__global__ void __launch_bounds__(256)
pl_clear(uint32_t* __restrict__ ctr) {
    for (int i = threadIdx.x; i < PL_C_COUNT; i += 256) ctr[i] = 0u;
}

static int pl_device_cus() {
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

bool dec_layer_ok(const DecodeArgs& a) {
    return a.s_up_t && a.s_dn_t && a.a_up_t && a.a_dn_t && a.T <= PL_T && a.R <= PL_RMAX &&
           a.d == 4096 && a.h % 1024 == 0 && a.h <= 16384 && a.r == KC &&
           (a.rL == 8 || a.rL == 16) && a.gq == KC && a.P <= 64 && a.G <= 64 && a.E <= 1024;
}

hipError_t launch_dec_layer(const DecodeArgs& a, hipStream_t s) {
    prof_begin(s);
    pl_clear<<<1, 256, 0, s>>>(a.pl_ctr);
    prof_end(s, "pl_clear");
    prof_begin(s);
    dec_layer<16><<<pl_device_cus(), PL_THREADS, 0, s>>>(a);
    prof_end(s, "dec_layer");
    return hipGetLastError();
}

}  // namespace em
