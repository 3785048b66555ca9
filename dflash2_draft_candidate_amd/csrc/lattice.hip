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
// One workgroup per position, built to keep the dependent global round trips at two:
//   1. candidate ids, predecessor ids, unary scores and the gate row (the gate arrives as
//      `ksplit` partial rows, summed here in split order);
//   2. the 2k codebook rows, gathered with 16-byte loads and widened into LDS as fp32, the
//      predecessor rows already multiplied by the gate (a chunk of the rank at a time when
//      2 k r floats would not fit).
// Each thread then accumulates its edges with fp32 FMA in rank order from float4 LDS reads.
// A predecessor or candidate id outside [0, V) yields NaN edges instead of an out-of-bounds read.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kLatThreads = 256;
constexpr int kMaxEdgesPerThread = 64 * 64 / kLatThreads;  // k <= 64

template <typename CB> struct Cb;
template <> struct Cb<float> {
    static constexpr int kVec = 4;
    static __device__ __forceinline__ float one(const float *p, int64_t i) { return p[i]; }
};
template <> struct Cb<uint16_t> {
    static constexpr int kVec = 8;
    static __device__ __forceinline__ float one(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
};

template <typename CB, bool VEC>
__global__ __launch_bounds__(kLatThreads) void lattice_kernel(
    const int32_t *__restrict__ cand_ids, const float *__restrict__ unary,
    const float *__restrict__ gpart, int ksplit, const CB *__restrict__ pred,
    const CB *__restrict__ succ, const int32_t *__restrict__ anchor, int L, int V, int r, int k,
    int dc, float *__restrict__ edges) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ int32_t prev_s[64], cand_s[64];
    __shared__ float u_s[64];
    __shared__ float g_s[256];
    const int pitch = VEC ? dc + 4 : dc + 1;  // float4-aligned rows, or odd pitch for scalar reads
    float *P = lds;                           // [k][pitch]: pred row * gate
    float *S = lds + k * pitch;               // [k][pitch]: succ row

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t R = gridDim.x;
    const int b = (int)(row / L), p = (int)(row % L);

    // Round trip 1: ids, unary, gate (independent of each other).
    if (tid < k) {
        prev_s[tid] = (p == 0) ? anchor[b] : cand_ids[(row - 1) * k + tid];
        cand_s[tid] = cand_ids[row * k + tid];
        u_s[tid] = unary[row * k + tid];
    }
    for (int d = tid; d < r; d += kLatThreads) {
        // the split partials are independent loads: issue 8 at a time, then add in split order
        float v = 0.f;
        for (int s = 0; s < ksplit; s += 8) {
            float part[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)  // clamped split index: unconditional loads
                part[q] = gpart[((int64_t)min(s + q, ksplit - 1) * R + row) * r + d];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (s + q < ksplit) v += part[q];
        }
        g_s[d] = v;
    }
    __syncthreads();

    const int kk = k * k;
    float acc[kMaxEdgesPerThread];
#pragma unroll
    for (int t = 0; t < kMaxEdgesPerThread; ++t) acc[t] = 0.f;

    for (int d0 = 0; d0 < r; d0 += dc) {
        const int dn = min(dc, r - d0);
        // Round trip 2: gather 2k codebook rows (columns d0 .. d0+dn) into LDS.
        if (VEC) {
            constexpr int NV = Cb<CB>::kVec;
            const int per_row = dn / NV;
            for (int t = tid; t < 2 * k * per_row; t += kLatThreads) {
                const int rr = t / per_row, d = (t % per_row) * NV;
                const bool is_succ = rr >= k;
                const int i = is_succ ? rr - k : rr;
                const int32_t id = is_succ ? cand_s[i] : prev_s[i];
                const bool ok = id >= 0 && id < V;
                // branch-free: an invalid id reads row 0 and is replaced by NaN afterwards
                const CB *src = (is_succ ? succ : pred) + (int64_t)(ok ? id : 0) * r + d0 + d;
                float v[NV];
                Elem<CB>::unpack(*reinterpret_cast<const u32x4 *>(src), v);
#pragma unroll
                for (int e = 0; e < NV; ++e) v[e] = ok ? v[e] : __builtin_nanf("");
                float *dst = (is_succ ? S : P) + i * pitch + d;
#pragma unroll
                for (int e = 0; e < NV; ++e) dst[e] = is_succ ? v[e] : v[e] * g_s[d0 + d + e];
            }
        } else {
            for (int t = tid; t < 2 * k * dn; t += kLatThreads) {
                const int rr = t / dn, d = t % dn;
                const bool is_succ = rr >= k;
                const int i = is_succ ? rr - k : rr;
                const int32_t id = is_succ ? cand_s[i] : prev_s[i];
                const bool ok = id >= 0 && id < V;
                float v = Cb<CB>::one(is_succ ? succ : pred, (int64_t)(ok ? id : 0) * r + d0 + d);
                v = ok ? v : __builtin_nanf("");
                (is_succ ? S : P)[i * pitch + d] = is_succ ? v : v * g_s[d0 + d];
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kMaxEdgesPerThread; ++t) {
            const int e = tid + t * kLatThreads;
            if (e < kk) {
                const float *pi = P + (e / k) * pitch;
                const float *sj = S + (e % k) * pitch;
                float a = acc[t];
                if (VEC) {
                    for (int d = 0; d < dn; d += 4) {
                        const float4 x = *reinterpret_cast<const float4 *>(pi + d);
                        const float4 y = *reinterpret_cast<const float4 *>(sj + d);
                        a = fmaf(x.x, y.x, a);
                        a = fmaf(x.y, y.y, a);
                        a = fmaf(x.z, y.z, a);
                        a = fmaf(x.w, y.w, a);
                    }
                } else {
                    for (int d = 0; d < dn; ++d) a = fmaf(pi[d], sj[d], a);
                }
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

template <typename CB>
hipError_t launch_cb(const int32_t *cand_ids, const float *unary, const float *gpart, int ksplit,
                     const void *pred_cb, const void *succ_cb, const int32_t *anchor_ids, int B,
                     int L, int V, int r, int k, float *edges, hipStream_t stream) {
    // Rank chunk: 2 k (dc + 4) floats of LDS stay under 48 KB.
    int dc = 6144 / k - 4;
    if (dc > r) dc = r;
    const bool vec = (r % Cb<CB>::kVec) == 0;
    if (vec) dc = dc / Cb<CB>::kVec * Cb<CB>::kVec;  // whole 16-byte vectors per chunk
    const size_t lds = (size_t)2 * k * (dc + 4) * sizeof(float);
    const dim3 grid((unsigned)((int64_t)B * L)), block(kLatThreads);
    const CB *pred = static_cast<const CB *>(pred_cb);
    const CB *succ = static_cast<const CB *>(succ_cb);
    if (vec)
        hipLaunchKernelGGL((lattice_kernel<CB, true>), grid, block, lds, stream, cand_ids, unary,
                           gpart, ksplit, pred, succ, anchor_ids, L, V, r, k, dc, edges);
    else
        hipLaunchKernelGGL((lattice_kernel<CB, false>), grid, block, lds, stream, cand_ids, unary,
                           gpart, ksplit, pred, succ, anchor_ids, L, V, r, k, dc, edges);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lattice(const int32_t *cand_ids, const float *unary, const float *gpart,
                          int ksplit, const void *pred_cb, const void *succ_cb, int cb_dtype,
                          const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                          float *edges, hipStream_t stream) {
    if (cb_dtype == 0)
        return launch_cb<float>(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb, anchor_ids, B, L,
                                V, r, k, edges, stream);
    return launch_cb<uint16_t>(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb, anchor_ids, B, L,
                               V, r, k, edges, stream);
}

}  // namespace dflash2
