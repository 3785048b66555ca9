// K2: the context gate g = hidden . W_sel (the selector's only dense contraction).
//
// Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path
// Selector" (the context gate H(h_t) applied to the predecessor embedding); "DFlash2 Lands in
// llama.cpp" (ramgpt.org), section "What llama.cpp Actually Builds for the Selector" (the current
// hidden state projected through the selector-hidden weight). Read here as a plain linear map.
//
// bf16 inputs run on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// The product is skinny (r <= 256 columns) and HBM-bound on reading `hidden`, so the kernel is
// built for independent loads in flight, with no LDS staging and no barriers in the main loop:
//   * a wave owns 16 rows and a range of H; the 4 waves of a workgroup split one range 4 ways
//     and are summed through LDS at the end; `splits` workgroups cover H;
//   * A fragments (8 consecutive h of one row) are 16-byte loads of `hidden`;
//   * W_sel is [H, r] (r contiguous), but a B fragment needs 8 consecutive h of one column. Each
//     lane loads 4-byte column pairs (2c, 2c+1) of its 8 rows of W_sel and repacks the low halves
//     into the fragment of one output tile and the high halves into the next, so the output
//     columns of tile pair (2p, 2p+1) at lane position m are 32p + 2m and 32p + 2m + 1. Every
//     load is independent: a batch of steps is issued before any MFMA runs;
//   * each split writes its own partial [R, r] tile; the lattice kernel (or, for the stand-alone
//     gate, a reduction kernel) sums the splits in split order: deterministic, no atomics.
// fp32 inputs use a plain fp32 FMA kernel that writes g directly.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 4;
constexpr int kGateThreads = kGateWaves * kWave;
constexpr int kStepK = 32;  // H per MFMA
constexpr int kTargetWgs = 256;

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// Output column of MFMA tile t at lane position m (NT >= 2: column pairs; NT == 1: identity).
template <int NT>
__device__ __forceinline__ int out_col(int t, int m) {
    return NT == 1 ? m : 32 * (t >> 1) + 2 * m + (t & 1);
}

template <int NT>
struct Step {
    static constexpr int NP = NT == 1 ? 1 : NT / 2;  // column pairs per lane
    u32x4 a;                                        // A fragment
    uint32_t w[8][NP];                              // W rows k0+8g+i, column pair p
};

// Loads of one 32-wide step. FAST (wave-uniform): the step lies inside H, H % 8 == 0 and r is
// exactly the padded tile width, so every load is unconditional (rows past R read row R-1 and
// are discarded at the store); no branch separates the loads, and they all stay in flight.
template <int NT, bool FAST>
__device__ __forceinline__ void load_step(Step<NT> &s, const uint16_t *hrow, bool row_ok,
                                          const uint16_t *W, int H, int r, int k0, int g, int m) {
    const int kc = k0 + 8 * g;
    if (FAST) {
        s.a = *reinterpret_cast<const u32x4 *>(hrow + kc);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t *wrow = W + (int64_t)(kc + i) * r;
#pragma unroll
            for (int p = 0; p < Step<NT>::NP; ++p)
                s.w[i][p] = NT == 1 ? (uint32_t)wrow[m]
                                    : *reinterpret_cast<const uint32_t *>(wrow + 32 * p + 2 * m);
        }
        return;
    }
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (row_ok && kc + i < H) ? hrow[kc + i] : 0u;
    s.a = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int kr = kc + i;
        const uint16_t *wrow = W + (int64_t)kr * r;
#pragma unroll
        for (int p = 0; p < Step<NT>::NP; ++p) {
            if (NT == 1) {
                s.w[i][p] = (kr < H && m < r) ? wrow[m] : 0u;
            } else {
                const int c = 32 * p + 2 * m;
                s.w[i][p] = (kr < H && c < r ? wrow[c] : 0u) |
                            ((kr < H && c + 1 < r ? (uint32_t)wrow[c + 1] : 0u) << 16);
            }
        }
    }
}

template <int NT>
__device__ __forceinline__ void mma_step(const Step<NT> &s, f32x4 *acc) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, s.a);
    if (NT == 1) {
        const u32x4 b = u32x4{lo_pair(s.w[0][0], s.w[1][0]), lo_pair(s.w[2][0], s.w[3][0]),
                              lo_pair(s.w[4][0], s.w[5][0]), lo_pair(s.w[6][0], s.w[7][0])};
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b), acc[0], 0, 0, 0);
        return;
    }
#pragma unroll
    for (int p = 0; p < Step<NT>::NP; ++p) {
        const u32x4 blo = u32x4{lo_pair(s.w[0][p], s.w[1][p]), lo_pair(s.w[2][p], s.w[3][p]),
                                lo_pair(s.w[4][p], s.w[5][p]), lo_pair(s.w[6][p], s.w[7][p])};
        const u32x4 bhi = u32x4{hi_pair(s.w[0][p], s.w[1][p]), hi_pair(s.w[2][p], s.w[3][p]),
                                hi_pair(s.w[4][p], s.w[5][p]), hi_pair(s.w[6][p], s.w[7][p])};
        acc[2 * p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, blo),
                                                             acc[2 * p], 0, 0, 0);
        acc[2 * p + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bhi),
                                                                 acc[2 * p + 1], 0, 0, 0);
    }
}

// Steps whose loads are issued together, by tile count (bounded by registers).
template <int NT> constexpr int batch_steps() { return NT <= 4 ? 4 : (NT == 8 ? 2 : 1); }

template <int NT>
__global__ __launch_bounds__(kGateThreads) void gate_bf16_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ W, int R, int H, int r,
    int splits, float *__restrict__ out) {
    constexpr int NC = NT * 16;
    constexpr int D = batch_steps<NT>();
    __shared__ float red[kGateWaves][16][NC + (NT == 16 ? 0 : 1)];  // <= 64 KB

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int m = lane & 15, g = lane >> 4;
    const int row = blockIdx.x * 16 + m;
    const bool row_ok = row < R;
    const uint16_t *hrow = hidden + (int64_t)(row_ok ? row : 0) * H;
    const bool vec_h = (H % 8) == 0;

    const int nsteps = (H + kStepK - 1) / kStepK;
    const int q = blockIdx.y * kGateWaves + wave, nq = splits * kGateWaves;
    const int s0 = (int)((int64_t)nsteps * q / nq), s1 = (int)((int64_t)nsteps * (q + 1) / nq);

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Full batches of D steps on the fast path; everything else (ragged H, odd r) step by step.
    const bool fast_ok = vec_h && r == NC;
    int s = s0;
    if (fast_ok) {
        for (; s + D <= s1 && (s + D) * kStepK <= H; s += D) {
            Step<NT> st[D];
#pragma unroll
            for (int d = 0; d < D; ++d)
                load_step<NT, true>(st[d], hrow, row_ok, W, H, r, (s + d) * kStepK, g, m);
#pragma unroll
            for (int d = 0; d < D; ++d) mma_step<NT>(st[d], acc);
        }
    }
    for (; s < s1; ++s) {
        Step<NT> st;
        load_step<NT, false>(st, hrow, row_ok, W, H, r, s * kStepK, g, m);
        mma_step<NT>(st, acc);
    }

    // acc[t][i]: row g*4+i of the tile, column out_col(t, m). Sum the 4 waves in order.
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][g * 4 + i][out_col<NT>(t, m)] = acc[t][i];
    __syncthreads();
    float *dst = out + (int64_t)blockIdx.y * R * r;
    for (int e = threadIdx.x; e < 16 * r; e += kGateThreads) {
        const int rr = e / r, c = e % r, orow = blockIdx.x * 16 + rr;
        if (orow >= R) continue;
        float v = red[0][rr][c];
#pragma unroll
        for (int w = 1; w < kGateWaves; ++w) v += red[w][rr][c];
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
__global__ __launch_bounds__(256) void gate_f32_kernel(const float *__restrict__ hidden,
                                                       const float *__restrict__ W, int R, int H,
                                                       int r, float *__restrict__ g) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)R * r) return;
    const int64_t row = e / r;
    const int c = (int)(e % r);
    const float *h = hidden + row * H;
    float acc = 0.f;
    for (int k = 0; k < H; ++k) acc = fmaf(h[k], W[(int64_t)k * r + c], acc);
    g[e] = acc;
}

template <int NT>
hipError_t launch_bf16(const uint16_t *hidden, const uint16_t *W, int R, int H, int r, int splits,
                       float *out, hipStream_t stream) {
    const dim3 grid((unsigned)((R + 15) / 16), (unsigned)splits);
    hipLaunchKernelGGL((gate_bf16_kernel<NT>), grid, dim3(kGateThreads), 0, stream, hidden, W, R,
                       H, r, splits, out);
    return hipGetLastError();
}

}  // namespace

int gate_splits(int R, int H, int act_dtype) {
    if (act_dtype == 0) return 1;
    const int64_t mtiles = (R + 15) / 16;
    const int64_t nsteps = (H + kStepK - 1) / kStepK;
    int64_t s = (kTargetWgs + mtiles - 1) / mtiles;
    const int64_t s_max = nsteps / kGateWaves;  // at least one step per wave
    if (s > s_max) s = s_max;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_gate_partials(const void *hidden, const void *W_sel, int act_dtype, int R,
                                int H, int r, float *part, hipStream_t stream) {
    if (act_dtype == 0) {
        const int64_t n = (int64_t)R * r;
        hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, static_cast<const float *>(hidden),
                           static_cast<const float *>(W_sel), R, H, r, part);
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
