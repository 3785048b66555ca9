// K2: the context gate g = hidden . W_sel (the selector's only dense contraction).
//
// Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path
// Selector" (the context gate H(h_t) applied to the predecessor embedding); "DFlash2 Lands in
// llama.cpp" (ramgpt.org), section "What llama.cpp Actually Builds for the Selector" (the current
// hidden state projected through the selector-hidden weight). Read here as a plain linear map.
//
// bf16 inputs run on the gfx950 matrix cores (gate_tile.h: v_mfma_f32_16x16x32_bf16, fp32
// accumulation). The product is skinny (r <= 256 columns) and HBM-bound on reading `hidden`, so
// the kernel is built for independent loads in flight, with no LDS staging and no barriers in
// the main loop:
//   * a wave owns 16 rows and a range of H; the 4 waves of a workgroup split one range 4 ways
//     and are summed through LDS at the end; `splits` workgroups cover H;
//   * each split writes its own partial [R, r] tile; the lattice kernel (or, for the stand-alone
//     gate, a reduction kernel) sums the splits in split order: deterministic, no atomics.
// The top-k kernel can compute the same tiles itself (one per workgroup, before it streams);
// the results are identical, since the waves' ranges and the summation order are the same.
// fp32 inputs use an fp32 FMA kernel (wave-wide dot products per output) that writes g
// directly.
#include "device_common.h"
#include "gate_tile.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kTargetWgs = 256;
constexpr int kMaxSplits = 8;  // the consumer adds at most this many partials, all loads at once

// Steps in flight per wave in the stand-alone kernel (a step holds 4 + 8 * max(1, NT / 2)
// registers): 8 (one round trip at H = 4096 with 4 splits) up to 8 column tiles, 4 at 16.
template <int NT> constexpr int kAloneSteps = NT <= 8 ? 8 : 4;

template <int NT>
__global__ __launch_bounds__(gate_waves<NT>() * kWave) void gate_bf16_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ W, int R, int H, int r,
    int splits, float *__restrict__ out) {
    constexpr int GW = gate_waves<NT>();
    __shared__ float red[GW][16][gate_pitch<NT>()];  // <= 64 KB

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int m = lane & 15, g = lane >> 4;
    int s0, s1;
    gate_steps(H, blockIdx.y * GW + wave, splits * GW, s0, s1);
    f32x4 acc[NT];
    // (alone, the kernel's registers allow more steps in flight than inside the top-k pass)
    gate_wave<NT, kAloneSteps<NT>, true>(hidden, W, R, H, r, blockIdx.x * 16, s0, s1, lane, acc);

    // acc[t][i]: row g*4+i of the tile, column out_col(t, m). Sum the GW waves in order.
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][g * 4 + i][out_col<NT>(t, m)] = acc[t][i];
    __syncthreads();
    float *dst = out + (int64_t)blockIdx.y * R * r;
    for (int e = threadIdx.x; e < 16 * r; e += GW * kWave) {
        const int rr = e / r, c = e % r, orow = blockIdx.x * 16 + rr;
        if (orow >= R) continue;
        float v = red[0][rr][c];
#pragma unroll
        for (int w = 1; w < GW; ++w) v += red[w][rr][c];
        dst[(int64_t)orow * r + c] = v;
    }
}

// g = sum over splits of the partial tiles, in split order (stand-alone gate only).
__global__ __launch_bounds__(256) void gate_reduce_kernel(const float *__restrict__ part,
                                                          int splits, int64_t n,
                                                          float *__restrict__ g) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float v = part[i];
    for (int s = 1; s < splits; ++s) v += part[(int64_t)s * n + i];
    g[i] = v;
}

// fp32 inputs: one output per thread, fp32 FMA over H in order.
// fp32 activations: one workgroup per row; wave w computes columns w, w + 4, ... as wave-wide
// dot products (lane L adds h[k] W[k][c] for k = L, L + 64, ... in order, then the 64 lane sums
// are added by a fixed tree), so a row costs one pass over H per column group instead of one
// thread running over H per output.
constexpr int kF32Waves = 4;

__global__ __launch_bounds__(kF32Waves * kWave) void gate_f32_kernel(
    const float *__restrict__ hidden, const float *__restrict__ W, int R, int H, int r,
    float *__restrict__ g) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = blockIdx.x;
    const float *h = hidden + row * H;
    for (int c = wave; c < r; c += kF32Waves) {
        float acc = 0.f;
        for (int k = lane; k < H; k += kWave) acc = fmaf(h[k], W[(int64_t)k * r + c], acc);
#pragma unroll
        for (int d = kWave / 2; d > 0; d /= 2) acc += __shfl_xor(acc, d, kWave);
        if (lane == 0) g[row * r + c] = acc;
    }
}

template <int NT>
hipError_t launch_bf16(const uint16_t *hidden, const uint16_t *W, int R, int H, int r, int splits,
                       float *out, hipStream_t stream) {
    const dim3 grid((unsigned)((R + 15) / 16), (unsigned)splits);
    hipLaunchKernelGGL((gate_bf16_kernel<NT>), grid, dim3(gate_waves<NT>() * kWave), 0, stream, hidden, W, R,
                       H, r, splits, out);
    return hipGetLastError();
}

}  // namespace

int gate_splits(int R, int H, int act_dtype) {
    if (act_dtype == 0) return 1;
    const int64_t mtiles = (R + 15) / 16;
    const int64_t nsteps = (H + kStepK - 1) / kStepK;
    int64_t s = (kTargetWgs + mtiles - 1) / mtiles;
    if (s > kMaxSplits) s = kMaxSplits;
    const int64_t s_max = nsteps / gate_waves<1>();  // at least one step per wave
    if (s > s_max) s = s_max;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_gate_partials(const void *hidden, const void *W_sel, int act_dtype, int R,
                                int H, int r, float *part, hipStream_t stream) {
    if (act_dtype == 0) {
        hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)R), dim3(kF32Waves * kWave), 0, stream,
                           static_cast<const float *>(hidden), static_cast<const float *>(W_sel),
                           R, H, r, part);
        return hipGetLastError();
    }
    const uint16_t *h = static_cast<const uint16_t *>(hidden);
    const uint16_t *w = static_cast<const uint16_t *>(W_sel);
    const int ks = gate_splits(R, H, act_dtype);
    const int nt = (r + 15) / 16;
    if (nt <= 1) return launch_bf16<1>(h, w, R, H, r, ks, part, stream);
    if (nt <= 2) return launch_bf16<2>(h, w, R, H, r, ks, part, stream);
    if (nt <= 4) return launch_bf16<4>(h, w, R, H, r, ks, part, stream);
    if (nt <= 8) return launch_bf16<8>(h, w, R, H, r, ks, part, stream);
    return launch_bf16<16>(h, w, R, H, r, ks, part, stream);
}

size_t gate_workspace_bytes(int R, int H, int r, int act_dtype) {
    const int ks = gate_splits(R, H, act_dtype);
    return ks > 1 ? (size_t)ks * R * r * sizeof(float) : 0;
}

hipError_t launch_gate(const void *hidden, const void *W_sel, int act_dtype, int R, int H, int r,
                       float *g, void *workspace, hipStream_t stream) {
    const int ks = gate_splits(R, H, act_dtype);
    if (ks == 1) return launch_gate_partials(hidden, W_sel, act_dtype, R, H, r, g, stream);
    float *part = static_cast<float *>(workspace);
    hipError_t e = launch_gate_partials(hidden, W_sel, act_dtype, R, H, r, part, stream);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)R * r;
    hipLaunchKernelGGL(gate_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       part, ks, n, g);
    return hipGetLastError();
}

}  // namespace dflash2
