// Token permutation (step a3): the T*k (token, slot) pairs sorted by expert and
// then token (hence also by group, since group = expert / P), the list of
// distinct tokens of each group sorted by token, and the maps between them.
//
// Method: one bit per (expert, token) and per (group, token).  Because a token
// never selects the same expert twice, an expert's rows in token order are
// exactly the set bits of its bitmap, so a prefix popcount over each bitmap row
// ranks every pair without sorting and without order-dependent atomics; the
// result is unique and reproducible.
#include "common.h"
#include "kernels.h"

namespace em {

__global__ void __launch_bounds__(256)
perm_clear(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

__global__ void __launch_bounds__(256)
perm_mark(const int32_t* __restrict__ idx, uint32_t* __restrict__ ebm,
          uint32_t* __restrict__ gbm, int T, int k, int P, int W) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= T * k) return;
    const int t = i / k;
    const int e = idx[i];
    const uint32_t bit = 1u << (t & 31);
    atomicOr(&ebm[(size_t)e * W + (t >> 5)], bit);
    atomicOr(&gbm[(size_t)(e / P) * W + (t >> 5)], bit);
}

// One workgroup per bitmap row (E expert rows, then G group rows): exclusive
// prefix popcount over the row's W words and the row total.
__global__ void __launch_bounds__(256)
perm_rank(const uint32_t* __restrict__ bm, uint32_t* __restrict__ pre,
          int32_t* __restrict__ total, int W) {
    __shared__ uint32_t part[256];
    const int row = blockIdx.x;
    const uint32_t* b = bm + (size_t)row * W;
    uint32_t* p = pre + (size_t)row * W;
    const int per = (W + 255) / 256;
    const int w0 = threadIdx.x * per;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i)
        if (w0 + i < W) s += __popc(b[w0 + i]);
    part[threadIdx.x] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan of 256 partial counts
    for (int off = 1; off < 256; off <<= 1) {
        uint32_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0u;
        __syncthreads();
        part[threadIdx.x] += v;
        __syncthreads();
    }
    uint32_t run = threadIdx.x ? part[threadIdx.x - 1] : 0u;
    for (int i = 0; i < per; ++i) {
        if (w0 + i < W) {
            p[w0 + i] = run;
            run += __popc(b[w0 + i]);
        }
    }
    if (threadIdx.x == 255) total[row] = (int32_t)part[255];
}

// Single workgroup: offsets of experts and groups and the per-segment m-tile
// prefixes used to map workgroups of the GEMM kernels onto segments (mt-row
// tiles for the general kernels, kPfTileRows-row tiles per expert for the
// tiled prefill GEMMs).
__global__ void __launch_bounds__(256)
perm_offsets(const int32_t* __restrict__ total, int E, int G, int P, int mt,
             int32_t* __restrict__ eoff, int32_t* __restrict__ uoff,
             int32_t* __restrict__ etile, int32_t* __restrict__ etile_pf, int32_t* __restrict__ gtile_u,
             int32_t* __restrict__ gtile_r) {
    __shared__ int srow[256], stile[256], stile2[256];
    __shared__ int s_eoff[1025];
    const int tid = threadIdx.x;
    const int per = (E + 255) / 256;         // <= 4
    int cr[4], ct[4], ct2[4], sr = 0, st = 0, st2 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * per + i;
        cr[i] = (i < per && e < E) ? total[e] : 0;
        ct[i] = (cr[i] + mt - 1) / mt;
        ct2[i] = (cr[i] + kPfTileRows - 1) / kPfTileRows;
        sr += cr[i];
        st += ct[i];
        st2 += ct2[i];
    }
    srow[tid] = sr;
    stile[tid] = st;
    stile2[tid] = st2;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int a = tid >= off ? srow[tid - off] : 0;
        const int b = tid >= off ? stile[tid - off] : 0;
        const int b2 = tid >= off ? stile2[tid - off] : 0;
        __syncthreads();
        srow[tid] += a;
        stile[tid] += b;
        stile2[tid] += b2;
        __syncthreads();
    }
    int ra = tid ? srow[tid - 1] : 0, ta = tid ? stile[tid - 1] : 0, ta2 = tid ? stile2[tid - 1] : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * per + i;
        if (i < per && e < E) {
            eoff[e] = ra;
            etile[e] = ta;
            etile_pf[e] = ta2;
            s_eoff[e] = ra;
            ra += cr[i];
            ta += ct[i];
            ta2 += ct2[i];
        }
    }
    if (tid == 255) {
        eoff[E] = srow[255];
        etile[E] = stile[255];
        etile_pf[E] = stile2[255];
        s_eoff[E] = srow[255];
    }
    __syncthreads();
    if (tid == 0) {
        int u = 0, tu = 0, tr = 0;
        for (int g = 0; g < G; ++g) {
            uoff[g] = u;
            gtile_u[g] = tu;
            gtile_r[g] = tr;
            const int c = total[E + g];
            u += c;
            tu += (c + mt - 1) / mt;
            const int rows = s_eoff[(g + 1) * P] - s_eoff[g * P];
            tr += (rows + mt - 1) / mt;
        }
        uoff[G] = u;
        gtile_u[G] = tu;
        gtile_r[G] = tr;
    }
}

// One thread per (bitmap row, word): emits the row records of every set bit.
__global__ void __launch_bounds__(256)
perm_emit(const int32_t* __restrict__ idx, const uint32_t* __restrict__ bm,
          const uint32_t* __restrict__ pre, const int32_t* __restrict__ eoff,
          const int32_t* __restrict__ uoff, int32_t* __restrict__ row_tok,
          int32_t* __restrict__ row_slot, int32_t* __restrict__ row_exp,
          int32_t* __restrict__ row_u, int32_t* __restrict__ slot_row,
          int32_t* __restrict__ ut_tok, int E, int G, int P, int k, int W) {
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;
    if (i >= (int64_t)(E + G) * W) return;
    const int row = (int)(i / W), w = (int)(i % W);
    uint32_t bits = bm[i];
    uint32_t rank = pre[i];
    if (row < E) {
        const int e = row, g = e / P;
        const uint32_t* gb = bm + (size_t)(E + g) * W;
        const uint32_t* gp = pre + (size_t)(E + g) * W;
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            const int t = w * 32 + b;
            const int r = eoff[e] + (int)rank++;
            int j = 0;
            for (; j < k; ++j)
                if (idx[(size_t)t * k + j] == e) break;
            row_tok[r] = t;
            row_slot[r] = j;
            row_exp[r] = e;
            slot_row[(size_t)t * k + j] = r;
            const uint32_t below = gb[w] & ((1u << b) - 1u);
            row_u[r] = uoff[g] + (int)(gp[w] + __popc(below));
        }
    } else {
        const int g = row - E;
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            ut_tok[uoff[g] + (int)rank++] = w * 32 + b;
        }
    }
}

hipError_t launch_dispatch(const int32_t* idx, const DispatchBufs& db, int T, int k, int E,
                           int P, int mt, hipStream_t stream) {
    const int G = E / P;
    const int W = (T + 31) / 32;
    const int64_t nbits = (int64_t)(E + G) * W;
    const int cgrid = (int)((nbits + 255) / 256 < 1024 ? (nbits + 255) / 256 : 1024);
    prof_begin(stream);
    perm_clear<<<cgrid, 256, 0, stream>>>(db.bm, nbits);
    prof_end(stream, "perm_clear");
    prof_begin(stream);
    perm_mark<<<(T * k + 255) / 256, 256, 0, stream>>>(idx, db.bm, db.bm + (size_t)E * W, T, k, P, W);
    prof_end(stream, "perm_mark");
    prof_begin(stream);
    perm_rank<<<E + G, 256, 0, stream>>>(db.bm, db.pre, db.total, W);
    prof_end(stream, "perm_rank");
    prof_begin(stream);
    perm_offsets<<<1, 256, 0, stream>>>(db.total, E, G, P, mt, db.eoff, db.uoff, db.etile, db.etile_pf,
                                       db.gtile_u, db.gtile_r);
    prof_end(stream, "perm_offsets");
    prof_begin(stream);
    perm_emit<<<(int)((nbits + 255) / 256), 256, 0, stream>>>(
        idx, db.bm, db.pre, db.eoff, db.uoff, db.row_tok, db.row_slot, db.row_exp, db.row_u,
        db.slot_row, db.ut_tok, E, G, P, k, W);
    prof_end(stream, "perm_emit");
    return hipGetLastError();
}

}  // namespace em
