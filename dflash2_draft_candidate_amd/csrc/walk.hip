// K4: the greedy walk through each sequence's lattice.
//
// j_0 = argmax_j edges[b][0][0][j]; j_p = argmax_j edges[b][p][j_{p-1}][j]; ties go to the lowest
// j; path[b][p] = cand_ids[b][p][j_p]. Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog),
// section "A Lightweight Path Selector" (the only sequential work: greedy follows the best
// successor from the last verified token); "DFlash2 Lands in llama.cpp" (ramgpt.org), section
// "What llama.cpp Actually Builds for the Selector" (the runtime walk: predecessor = anchor, best
// successor per position, emit the chosen token).
//
// The walk only ever needs, for each position p and predecessor i, the chosen successor
// best[p][i]; all of those are independent. So one workgroup per sequence stages a chunk of
// positions (edges and candidate ids) in LDS with coalesced loads, computes every best[p][i] in
// parallel (one row per thread), and only the final pointer chase j_p = best[p][j_{p-1}] is
// sequential: one LDS read per position.
//
// Two further modes. Sampling at temperature T > 0 (same blog section: sampling draws from the
// same scores): j is drawn from softmax(row / T) by inverse CDF from the caller's uniform
// u[b][p] (one per position, so every row of the position can draw in parallel): the smallest j
// whose running sum of w_j = 2^((e_j - m) log2e / T) exceeds u * sum_j w_j, in index order.
// Early stop ("DFlash2 Lands in llama.cpp", section "p_min Means Something Different Under
// DFlash2"): the confidence of a row at its choice j is exp(e_j - m) / sum_i exp(e_i - m); the
// drafted block ends before the first position whose chosen row's confidence is below p_min
// (draft_len), while the walk itself runs to the end.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kWalkThreads = 256;
constexpr int kWalkLds = 8192;  // floats of staged lattice (32 KB)

__global__ __launch_bounds__(kWalkThreads) void walk_kernel(
    const float *__restrict__ edges, const int32_t *__restrict__ cand_ids, int L, int k,
    float temperature, const float *__restrict__ uniforms, float p_min,
    int32_t *__restrict__ path, int32_t *__restrict__ path_idx, int32_t *__restrict__ draft_len) {
    __shared__ __attribute__((aligned(16))) float E[kWalkLds];
    __shared__ int32_t C[kWalkLds / 2];
    __shared__ int32_t best[kWalkLds / 2];
    __shared__ float conf[kWalkLds / 2];
    const bool sample = temperature > 0.f;
    const float scale = sample ? kLog2e / temperature : 0.f;
    int stop = L;
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
        // the choice of every (position, predecessor) row: greedy takes the lowest index among
        // the maxima; sampling inverts the running sum of the row's weights
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
            const float m = bv;
            if (sample) {
                float total = 0.f;
                for (int j = 0; j < k; ++j) total += __builtin_amdgcn_exp2f((rowp[j] - m) * scale);
                const float target = uniforms[row0 + t / k] * total;
                float run = 0.f;
                int pick = -1, last = 0;
                for (int j = 0; j < k; ++j) {
                    const float wj = __builtin_amdgcn_exp2f((rowp[j] - m) * scale);
                    run += wj;
                    if (pick < 0 && run > target) pick = j;
                    if (wj != 0.f) last = j;
                }
                bj = pick >= 0 ? pick : last;
            }
            if (p_min > 0.f) {
                float z = 0.f;
                for (int j = 0; j < k; ++j) z += __builtin_amdgcn_exp2f((rowp[j] - m) * kLog2e);
                conf[t] = __builtin_amdgcn_exp2f((rowp[bj] - m) * kLog2e) / z;
            }
            best[t] = bj;
        }
        __syncthreads();
        if (tid == 0) {
            for (int q = 0; q < np; ++q) {
                const int j = best[q * k + prev];
                path[row0 + q] = C[q * k + j];
                if (path_idx) path_idx[row0 + q] = j;
                if (p_min > 0.f && stop == L && conf[q * k + prev] < p_min) stop = p0 + q;
                prev = j;
            }
        }
    }
    if (tid == 0 && draft_len) draft_len[b] = stop;
}

}  // namespace

hipError_t launch_walk(const float *edges, const int32_t *cand_ids, int B, int L, int k,
                       int32_t *path, int32_t *path_idx, hipStream_t stream,
                       const WalkMode *mode) {
    const WalkMode greedy{};
    const WalkMode &md = mode ? *mode : greedy;
    hipLaunchKernelGGL(walk_kernel, dim3((unsigned)B), dim3(kWalkThreads), 0, stream, edges,
                       cand_ids, L, k, md.temperature, md.uniforms, md.p_min, path, path_idx,
                       md.draft_len);
    return hipGetLastError();
}

}  // namespace dflash2
