// K2: the context gate g = hidden . W_sel (the selector's only dense contraction).
//
// Source: "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path
// Selector" (the context gate H(h_t) applied to the predecessor embedding); "DFlash2 Lands in
// llama.cpp" (ramgpt.org), section "What llama.cpp Actually Builds for the Selector" (the current
// hidden state projected through the selector-hidden weight). Read here as a plain linear map.
//
// bf16 inputs run on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   * a workgroup owns 16 rows of hidden and one of `ksplit` ranges of H; its 4 waves split that
//     range again and each accumulates a 16 x (16*NT) tile of g;
//   * A fragments (hidden) are read straight from HBM, 16 bytes per lane; W_sel is [H, r]
//     (r contiguous), so each wave stages its 32 x r slab in LDS transposed to [r][32], which
//     turns every B fragment into one 16-byte LDS read;
//   * the 4 wave tiles are summed in fixed order through LDS; with ksplit > 1 the partial tiles go
//     to the workspace and a second kernel sums them in split order (deterministic, no atomics).
// fp32 inputs use a plain fp32 FMA kernel.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 4;
constexpr int kStepK = 32;  // H consumed per MFMA step

template <int NT>
__global__ __launch_bounds__(kGateWaves *kWave) void gate_bf16_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ W, int R, int H, int r,
    int ksplit, float *__restrict__ out) {
    constexpr int NC = NT * 16;  // padded output columns
    __shared__ __attribute__((aligned(16))) uint16_t smem[kGateWaves * NC * kStepK];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int m0 = blockIdx.x * 16;
    const int nsteps = (H + kStepK - 1) / kStepK;
    const int q = blockIdx.y * kGateWaves + wave, nq = ksplit * kGateWaves;
    const int s0 = (int)((int64_t)nsteps * q / nq), s1 = (int)((int64_t)nsteps * (q + 1) / nq);

    const int arow = m0 + (lane & 15);
    const int kg = (lane >> 4) * 8;
    const bool vec_h = (H % 8) == 0;
    const bool vec_r = (r % 8) == 0;
    constexpr int NV = NC / 8;  // 8-column chunks of the slab
    uint16_t *T = smem + wave * NC * kStepK;

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int step = s0; step < s1; ++step) {
        const int k0 = step * kStepK;
        // A fragment: row arow, k0 + kg .. +8
        u32x4 a_raw = u32x4{0u, 0u, 0u, 0u};
        if (arow < R) {
            const uint16_t *src = hidden + (int64_t)arow * H + k0 + kg;
            if (vec_h && k0 + kg + 8 <= H) {
                a_raw = *reinterpret_cast<const u32x4 *>(src);
            } else {
                uint16_t v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (k0 + kg + i < H) ? src[i] : (uint16_t)0;
                a_raw = u32x4{v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                              v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
            }
        }
        // W slab rows k0 .. k0+31, all columns, transposed into T[n][kk].
        for (int c = lane; c < kStepK * NV; c += kWave) {
            const int kk = c / NV, n0 = (c % NV) * 8, kgl = k0 + kk;
            uint16_t v[8];
            if (kgl < H && vec_r && n0 + 8 <= r) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(W + (int64_t)kgl * r + n0);
                v[0] = (uint16_t)w.x; v[1] = (uint16_t)(w.x >> 16);
                v[2] = (uint16_t)w.y; v[3] = (uint16_t)(w.y >> 16);
                v[4] = (uint16_t)w.z; v[5] = (uint16_t)(w.z >> 16);
                v[6] = (uint16_t)w.w; v[7] = (uint16_t)(w.w >> 16);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[i] = (kgl < H && n0 + i < r) ? W[(int64_t)kgl * r + n0 + i] : (uint16_t)0;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) T[(n0 + i) * kStepK + kk] = v[i];
        }
        const bf16x8 a = __builtin_bit_cast(bf16x8, a_raw);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const u32x4 b_raw =
                *reinterpret_cast<const u32x4 *>(T + (t * 16 + (lane & 15)) * kStepK + kg);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b_raw),
                                                             acc[t], 0, 0, 0);
        }
    }

    // Sum the 4 wave tiles in wave order.
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);  // [4][16][NC] floats: same bytes as the slabs
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[(wave * 16 + (lane >> 4) * 4 + i) * NC + t * 16 + (lane & 15)] = acc[t][i];
    __syncthreads();
    float *dst = out + (int64_t)blockIdx.y * R * r;
    for (int e = threadIdx.x; e < 16 * r; e += kGateWaves * kWave) {
        const int rr = e / r, c = e % r, row = m0 + rr;
        if (row >= R) continue;
        float v = red[rr * NC + c];
#pragma unroll
        for (int w = 1; w < kGateWaves; ++w) v += red[(w * 16 + rr) * NC + c];
        dst[(int64_t)row * r + c] = v;
    }
}

// g = sum over splits of the partial tiles, in split order.
__global__ __launch_bounds__(256) void gate_reduce_kernel(const float *__restrict__ part,
                                                          int ksplit, int64_t n,
                                                          float *__restrict__ g) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float v = part[i];
    for (int s = 1; s < ksplit; ++s) v += part[(int64_t)s * n + i];
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
hipError_t launch_bf16(const GatePlan &plan, const uint16_t *hidden, const uint16_t *W, int R,
                       int H, int r, float *g, float *part, hipStream_t stream) {
    const dim3 grid((unsigned)((R + 15) / 16), (unsigned)plan.ksplit);
    float *dst = plan.ksplit > 1 ? part : g;
    hipLaunchKernelGGL((gate_bf16_kernel<NT>), grid, dim3(kGateWaves * kWave), 0, stream, hidden,
                       W, R, H, r, plan.ksplit, dst);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.ksplit == 1) return e;
    const int64_t n = (int64_t)R * r;
    hipLaunchKernelGGL(gate_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       part, plan.ksplit, n, g);
    return hipGetLastError();
}

}  // namespace

GatePlan plan_gate(int R, int H, int r) {
    (void)r;
    GatePlan p;
    const int64_t mtiles = (R + 15) / 16;
    const int64_t nsteps = (H + kStepK - 1) / kStepK;
    int64_t ks = (1024 + mtiles - 1) / mtiles;           // about 1024 workgroups
    const int64_t ks_max = nsteps / (2 * kGateWaves);      // at least 2 steps per wave
    if (ks > ks_max) ks = ks_max;
    if (ks < 1) ks = 1;
    p.ksplit = (int)ks;
    return p;
}

size_t gate_workspace_bytes(const GatePlan &p, int R, int r) {
    return p.ksplit > 1 ? (size_t)p.ksplit * R * r * sizeof(float) : 0;
}

hipError_t launch_gate(const void *hidden, const void *W_sel, int act_dtype, int R, int H, int r,
                       float *g, void *workspace, hipStream_t stream) {
    if (act_dtype == 0) {
        const int64_t n = (int64_t)R * r;
        hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, static_cast<const float *>(hidden),
                           static_cast<const float *>(W_sel), R, H, r, g);
        return hipGetLastError();
    }
    const GatePlan plan = plan_gate(R, H, r);
    const uint16_t *h = static_cast<const uint16_t *>(hidden);
    const uint16_t *w = static_cast<const uint16_t *>(W_sel);
    float *part = static_cast<float *>(workspace);
    const int nt = (r + 15) / 16;
    if (nt <= 1) return launch_bf16<1>(plan, h, w, R, H, r, g, part, stream);
    if (nt <= 2) return launch_bf16<2>(plan, h, w, R, H, r, g, part, stream);
    if (nt <= 4) return launch_bf16<4>(plan, h, w, R, H, r, g, part, stream);
    if (nt <= 8) return launch_bf16<8>(plan, h, w, R, H, r, g, part, stream);
    return launch_bf16<16>(plan, h, w, R, H, r, g, part, stream);
}

}  // namespace dflash2
