// K4: the greedy walk through each sequence's lattice.
//
// j_0 = argmax_j edges[b][0][0][j]; j_p = argmax_j edges[b][p][j_{p-1}][j]; ties go to the lowest
// j; path[b][p] = cand_ids[b][p][j_p]. Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog),
// section "A Lightweight Path Selector" (the only sequential work: greedy follows the best
// successor from the last verified token); "DFlash2 Lands in llama.cpp" (ramgpt.org), section
// "What llama.cpp Actually Builds for the Selector" (the runtime walk: predecessor = anchor, best
// successor per position, emit the chosen token).
//
// One workgroup per sequence. The lattice is staged into LDS a chunk of positions at a time
// (coalesced, all 4 waves), then wave 0 walks it: lane j holds edge j of the current row and a
// 6-step butterfly finds the (value, lowest index) maximum.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kWalkThreads = 256;
constexpr int kWalkLds = 8192;  // floats of staged lattice (32 KB)

__global__ __launch_bounds__(kWalkThreads) void walk_kernel(const float *__restrict__ edges,
                                                            const int32_t *__restrict__ cand_ids,
                                                            int L, int k,
                                                            int32_t *__restrict__ path,
                                                            int32_t *__restrict__ path_idx) {
    __shared__ float E[kWalkLds];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t b = blockIdx.x;
    const int per_pos = k * k;
    const int chunk = kWalkLds / per_pos;  // >= 2 for k <= 64
    int prev = 0;
    for (int p0 = 0; p0 < L; p0 += chunk) {
        const int np = min(chunk, L - p0);
        __syncthreads();
        const float *src = edges + (b * L + p0) * per_pos;
        for (int e = tid; e < np * per_pos; e += kWalkThreads) E[e] = src[e];
        __syncthreads();
        if (wave != 0) continue;
        for (int q = 0; q < np; ++q) {
            float v = lane < k ? E[q * per_pos + prev * k + lane] : -INFINITY;
            int j = lane;
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) {
                const float ov = __shfl_xor(v, off, kWave);
                const int oj = __shfl_xor(j, off, kWave);
                if (ov > v || (ov == v && oj < j)) {
                    v = ov;
                    j = oj;
                }
            }
            j = __builtin_amdgcn_readfirstlane(j);
            j = j < k ? j : k - 1;
            const int64_t row = b * L + p0 + q;
            if (lane == 0) {
                path[row] = cand_ids[row * k + j];
                if (path_idx) path_idx[row] = j;
            }
            prev = j;
        }
    }
}

}  // namespace

hipError_t launch_walk(const float *edges, const int32_t *cand_ids, int B, int L, int k,
                       int32_t *path, int32_t *path_idx, hipStream_t stream) {
    hipLaunchKernelGGL(walk_kernel, dim3((unsigned)B), dim3(kWalkThreads), 0, stream, edges,
                       cand_ids, L, k, path, path_idx);
    return hipGetLastError();
}

}  // namespace dflash2
