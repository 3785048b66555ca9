// K3 (+ K4): the k x k transition lattice of every draft position, and the greedy walk. The
// computation and its sources are in lattice_body.h; this file launches it, one workgroup per
// sequence (with the walk) or per pass of positions.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "lattice_body.h"

namespace dflash2 {
namespace {

// Grid (B, passes): workgroup (b, c) covers positions of sequence b; with WALK it covers all of
// them (c = 0) pass by pass, else pass c only. pp positions per pass, KT waves per position.
// Dynamic LDS: the gate rows, [waves][rpad] floats.
// ONE (with WALK): the block is a single pass (L <= pp), known at compile time.
template <typename CB, int KT, bool WALK, bool ONE>
__global__ __launch_bounds__(lat_waves(KT, sizeof(CB)) * kWave) void lattice_kernel(LatArgs<CB> a) {
    extern __shared__ __attribute__((aligned(16))) float gsh[];
    __shared__ LatShared<WALK> ls;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    lattice_sequence<CB, KT, WALK, false, ONE>(a, (int)blockIdx.x, (int)blockIdx.y, wave, lane, ls,
                                               gsh);
}

// Positions per pass for k and codebook element size cb: every wave of a workgroup busy.
int positions_per_pass(int L, int k, int cb) {
    const int kt = (k + 15) / 16;
    const int KT = kt == 3 ? 4 : kt;
    const int pp = lat_waves(KT, cb) / KT;
    return L < pp ? L : pp;
}

template <typename CB, int KT, bool WALK>
void launch_kt(dim3 grid, int waves, size_t lds, hipStream_t stream, const LatArgs<CB> &a) {
    if constexpr (WALK) {
        if (a.L <= a.pp) {
            hipLaunchKernelGGL((lattice_kernel<CB, KT, true, true>), grid, dim3(waves * kWave), lds,
                               stream, a);
            return;
        }
    }
    hipLaunchKernelGGL((lattice_kernel<CB, KT, WALK, false>), grid, dim3(waves * kWave), lds,
                       stream, a);
}

template <typename CB, bool WALK>
hipError_t launch_cb(const int32_t *cand_ids, const float *unary, const float *gpart, int ksplit,
                     const void *pred_cb, const void *succ_cb, const int32_t *anchor_ids, int B,
                     int L, int V, int r, int k, float *edges, int32_t *path, int32_t *path_idx,
                     float p_min, int32_t *draft_len, hipStream_t stream) {
    const int kt = (k + 15) / 16;
    const int KT = kt == 3 ? 4 : kt;
    const int pp = positions_per_pass(L, k, sizeof(CB));
    const int waves = pp * KT;
    const int rpad = (r + kRankChunk - 1) / kRankChunk * kRankChunk;
    const size_t lds = (size_t)waves * rpad * sizeof(float);
    const dim3 grid((unsigned)B, WALK ? 1u : (unsigned)((L + pp - 1) / pp));
    const CB *pred = static_cast<const CB *>(pred_cb);
    const CB *succ = static_cast<const CB *>(succ_cb);
    const LatArgs<CB> a{cand_ids, unary, gpart, ksplit, pred, succ, anchor_ids, B, L, V, r, k,
                        pp, edges, path, path_idx, p_min, draft_len};
    auto go = [&](auto kernel_tag) {
        constexpr int K = decltype(kernel_tag)::value;
        launch_kt<CB, K, WALK>(grid, waves, lds, stream, a);
    };
    if (KT == 1)
        go(std::integral_constant<int, 1>{});
    else if (KT == 2)
        go(std::integral_constant<int, 2>{});
    else
        go(std::integral_constant<int, 4>{});
    return hipGetLastError();
}

}  // namespace

bool lattice_walk_fits(int L, int k, int cb_dtype) {
    const int pp = positions_per_pass(L, k, cb_dtype == 0 ? 4 : 2);
    return (L + pp - 1) / pp <= kMaxPasses;
}

hipError_t launch_lattice(const int32_t *cand_ids, const float *unary, const float *gpart,
                          int ksplit, const void *pred_cb, const void *succ_cb, int cb_dtype,
                          const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                          float *edges, hipStream_t stream) {
    if (cb_dtype == 0)
        return launch_cb<float, false>(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb,
                                       anchor_ids, B, L, V, r, k, edges, nullptr, nullptr, 0.f,
                                       nullptr, stream);
    return launch_cb<uint16_t, false>(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb, anchor_ids,
                                      B, L, V, r, k, edges, nullptr, nullptr, 0.f, nullptr,
                                      stream);
}

hipError_t launch_lattice_walk(const int32_t *cand_ids, const float *unary, const float *gpart,
                               int ksplit, const void *pred_cb, const void *succ_cb, int cb_dtype,
                               const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                               float *edges, int32_t *path, int32_t *path_idx, float p_min,
                               int32_t *draft_len, hipStream_t stream) {
    if (cb_dtype == 0)
        return launch_cb<float, true>(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb, anchor_ids,
                                      B, L, V, r, k, edges, path, path_idx, p_min, draft_len,
                                      stream);
    return launch_cb<uint16_t, true>(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb, anchor_ids,
                                     B, L, V, r, k, edges, path, path_idx, p_min, draft_len,
                                     stream);
}

}  // namespace dflash2
