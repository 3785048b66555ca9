// K3: the k x k transition lattice of every draft position.
//
// edges[b][p][i][j] = unary[b][p][j] + sum_d pred_cb[prev_i][d] * succ_cb[cand_j][d] * g[b][p][d]
// with prev_i = anchor_ids[b] at p = 0 and cand_ids[b][p-1][i] after. Source: "DFlash 2: Keep
// Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector", eq.
// S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>; "DFlash2 Lands in llama.cpp" (ramgpt.org), section
// "What llama.cpp Actually Builds for the Selector" (successor rows of the current candidates,
// predecessor rows of the previous ones, the hidden gate of the current position; the anchor is
// the first predecessor).
//
// One workgroup per position: the k predecessor rows (already multiplied by the gate) and the k
// successor rows are gathered into LDS as fp32, a chunk of the rank at a time, and each thread
// accumulates its edges with fp32 FMA in rank order. A predecessor or candidate id outside
// [0, V) yields NaN for the affected edges instead of an out-of-bounds read.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kLatThreads = 256;
constexpr int kMaxEdgesPerThread = 64 * 64 / kLatThreads;  // k <= 64

template <typename CB> __device__ __forceinline__ float cb_value(const CB *p, int64_t i);
template <> __device__ __forceinline__ float cb_value<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float cb_value<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

template <typename CB>
__global__ __launch_bounds__(kLatThreads) void lattice_kernel(
    const int32_t *__restrict__ cand_ids, const float *__restrict__ unary,
    const float *__restrict__ g, const CB *__restrict__ pred, const CB *__restrict__ succ,
    const int32_t *__restrict__ anchor, int L, int V, int r, int k, int dc,
    float *__restrict__ edges) {
    extern __shared__ float lds[];
    __shared__ int32_t prev_s[64], cand_s[64];
    __shared__ float u_s[64];
    const int dcp = dc + 1;  // padded row stride
    float *P = lds;          // [k][dcp]
    float *S = lds + k * dcp;

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / L), p = (int)(row % L);
    if (tid < k) {
        prev_s[tid] = (p == 0) ? anchor[b] : cand_ids[(row - 1) * k + tid];
        cand_s[tid] = cand_ids[row * k + tid];
        u_s[tid] = unary[row * k + tid];
    }
    __syncthreads();

    const int kk = k * k;
    float acc[kMaxEdgesPerThread];
#pragma unroll
    for (int t = 0; t < kMaxEdgesPerThread; ++t) acc[t] = 0.f;

    for (int d0 = 0; d0 < r; d0 += dc) {
        const int dn = min(dc, r - d0);
        for (int e = tid; e < k * dn; e += kLatThreads) {
            const int i = e / dn, d = e % dn;
            const int32_t pv = prev_s[i], cv = cand_s[i];
            P[i * dcp + d] = (pv >= 0 && pv < V)
                                 ? cb_value(pred, (int64_t)pv * r + d0 + d) * g[row * r + d0 + d]
                                 : __builtin_nanf("");
            S[i * dcp + d] = (cv >= 0 && cv < V) ? cb_value(succ, (int64_t)cv * r + d0 + d)
                                                 : __builtin_nanf("");
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kMaxEdgesPerThread; ++t) {
            const int e = tid + t * kLatThreads;
            if (e < kk) {
                const float *pi = P + (e / k) * dcp;
                const float *sj = S + (e % k) * dcp;
                float a = acc[t];
                for (int d = 0; d < dn; ++d) a = fmaf(pi[d], sj[d], a);
                acc[t] = a;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < kMaxEdgesPerThread; ++t) {
        const int e = tid + t * kLatThreads;
        if (e < kk) edges[row * kk + e] = u_s[e % k] + acc[t];
    }
}

}  // namespace

hipError_t launch_lattice(const int32_t *cand_ids, const float *unary, const float *g,
                          const void *pred_cb, const void *succ_cb, int cb_dtype,
                          const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                          float *edges, hipStream_t stream) {
    int dc = 4096 / k;  // rank chunk: 2 * k * (dc + 1) floats of LDS, at most ~33 KB
    if (dc > r) dc = r;
    const size_t lds = (size_t)2 * k * (dc + 1) * sizeof(float);
    const dim3 grid((unsigned)((int64_t)B * L)), block(kLatThreads);
    if (cb_dtype == 0)
        hipLaunchKernelGGL(lattice_kernel<float>, grid, block, lds, stream, cand_ids, unary, g,
                           static_cast<const float *>(pred_cb), static_cast<const float *>(succ_cb),
                           anchor_ids, L, V, r, k, dc, edges);
    else
        hipLaunchKernelGGL(lattice_kernel<uint16_t>, grid, block, lds, stream, cand_ids, unary, g,
                           static_cast<const uint16_t *>(pred_cb),
                           static_cast<const uint16_t *>(succ_cb), anchor_ids, L, V, r, k, dc,
                           edges);
    return hipGetLastError();
}

}  // namespace dflash2
