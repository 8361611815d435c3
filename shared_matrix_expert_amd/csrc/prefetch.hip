// Next-layer prefetch of the shared matrices (the prerouter idea).
//
// The launch post and the byteiota page describe a light head that predicts
// the next layer's routing one token ahead, so that the experts it will need
// can be fetched while the current layer computes (byteiota "Edge0-145B: Run a
// 145B Open-Source Model on Your Laptop", The Three Pillars, Prerouter
// paragraph; the Chinese commentary page, "145B 为什么不用同时装进显存").
// On one MI355X every weight is already in HBM; the tier that a prediction can
// still fill is the 256 MB memory-side cache (Infinity Cache) in front of
// HBM.  This kernel reads the predicted groups' shared matrices (int4 codes
// and scales) once, so that the next layer's first kernels find them there;
// it computes nothing and changes no result.  Which groups to read comes from
// the caller (a predictor); wrong or duplicate entries only waste bandwidth,
// and entries outside 0..G-1 are skipped.
#include "common.h"
#include "kernels.h"

namespace em {

// Workgroups stride over (listed group, 32 KB piece) pairs of one region;
// every lane loads eight 16-byte pieces per turn (all in flight together) and
// folds them into one word, which it writes to `sink` (one word per thread of
// the grid) so that no load is dropped.
constexpr int PF_LANES = 256;
constexpr size_t PF_PIECE = 8 * 16 * PF_LANES;

__global__ void __launch_bounds__(PF_LANES)
prefetch_groups(const uint8_t* __restrict__ base, size_t group_bytes, const int32_t* __restrict__ groups,
                int n_groups, int G, uint32_t* __restrict__ sink) {
    const size_t pieces = (group_bytes + PF_PIECE - 1) / PF_PIECE;
    const size_t total = pieces * (size_t)n_groups;
    uint32_t fold = 0;
    for (size_t p = blockIdx.x; p < total; p += gridDim.x) {
        const int g = groups[p / pieces];
        if (g < 0 || g >= G) continue;
        const size_t off = (p % pieces) * PF_PIECE;
        const uint8_t* src = base + (size_t)g * group_bytes + off;
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const size_t o = (size_t)(threadIdx.x + PF_LANES * i) * 16;
            v[i] = off + o + 16 <= group_bytes ? *reinterpret_cast<const uint4*>(src + o) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) fold ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    sink[(size_t)blockIdx.x * PF_LANES + threadIdx.x] = fold;
}

hipError_t launch_prefetch(const uint8_t* const* bases, const size_t* group_bytes, int n_regions,
                           const int32_t* groups, int n_groups, int G, uint32_t* sink, int blocks, hipStream_t s) {
    for (int i = 0; i < n_regions; ++i) {
        prof_begin(s);
        prefetch_groups<<<blocks, 256, 0, s>>>(bases[i], group_bytes[i], groups, n_groups, G, sink);
        prof_end(s, "prefetch_groups");
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace em
