// K4: the greedy walk through each sequence's lattice.
//
// j_0 = argmax_j edges[b][0][0][j]; j_p = argmax_j edges[b][p][j_{p-1}][j]; ties go to the lowest
// j; path[b][p] = cand_ids[b][p][j_p]. Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog),
// section "A Lightweight Path Selector" (the only sequential work: greedy follows the best
// successor from the last verified token); "DFlash2 Lands in llama.cpp" (ramgpt.org), section
// "What llama.cpp Actually Builds for the Selector" (the runtime walk: predecessor = anchor, best
// successor per position, emit the chosen token).
//
// The walk only ever needs, for each position p and predecessor i, the best successor
// best[p][i] = argmax_j edges[b][p][i][j]; all of those are independent. So one workgroup per
// sequence stages a chunk of positions (edges and candidate ids) in LDS with coalesced loads,
// computes every best[p][i] in parallel (one row per thread), and only the final pointer chase
// j_p = best[p][j_{p-1}] is sequential: one LDS read per position.
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
    __shared__ __attribute__((aligned(16))) float E[kWalkLds];
    __shared__ int32_t C[kWalkLds / 2];
    __shared__ int32_t best[kWalkLds / 2];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int per_pos = k * k;
    const int chunk = min(kWalkLds / per_pos, (kWalkLds / 2) / k);  // >= 2 for k <= 64
    int prev = 0;
    for (int p0 = 0; p0 < L; p0 += chunk) {
        const int np = min(chunk, L - p0);
        __syncthreads();
        const int64_t row0 = b * L + p0;
        const float *src = edges + row0 * per_pos;
        const int ne = np * per_pos;
        // Staging loads are issued in batches of 8 per thread before any LDS store, so they are
        // in flight together (at most 8192 floats: 8 float4 per thread).
        if (((row0 * per_pos) & 3) == 0 && (ne & 3) == 0) {  // 16-byte aligned run
            const float4 *s4 = reinterpret_cast<const float4 *>(src);
            float4 *e4 = reinterpret_cast<float4 *>(E);
            float4 t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = tid + u * kWalkThreads;
                t[u] = s4[e < ne / 4 ? e : 0];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = tid + u * kWalkThreads;
                if (e < ne / 4) e4[e] = t[u];
            }
        } else {
            for (int e0 = 0; e0 < ne; e0 += 8 * kWalkThreads) {
                float t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + tid + u * kWalkThreads;
                    t[u] = src[e < ne ? e : 0];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + tid + u * kWalkThreads;
                    if (e < ne) E[e] = t[u];
                }
            }
        }
        for (int e0 = 0; e0 < np * k; e0 += 4 * kWalkThreads) {
            int32_t t[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + tid + u * kWalkThreads;
                t[u] = cand_ids[row0 * k + (e < np * k ? e : 0)];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + tid + u * kWalkThreads;
                if (e < np * k) C[e] = t[u];
            }
        }
        __syncthreads();
        // best successor of every (position, predecessor) row: lowest index among the maxima
        for (int t = tid; t < np * k; t += kWalkThreads) {
            const float *rowp = E + t * k;
            float bv = rowp[0];
            int bj = 0;
            for (int j = 1; j < k; ++j) {
                const float v = rowp[j];
                if (v > bv) {
                    bv = v;
                    bj = j;
                }
            }
            best[t] = bj;
        }
        __syncthreads();
        if (tid == 0) {
            for (int q = 0; q < np; ++q) {
                const int j = best[q * k + prev];
                path[row0 + q] = C[q * k + j];
                if (path_idx) path_idx[row0 + q] = j;
                prev = j;
            }
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
