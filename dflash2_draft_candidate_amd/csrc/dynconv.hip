// The grouped dynamic depthwise convolution of the draft blocks.
//
// y[b][t][c] = sum_{tap < K} (base[tap][c] + dyn[b][t][tap][c / G]) * x[b][t - tap][c], with
// x[b][t'][c] = 0 for t' < 0: nothing crosses a block boundary. Sources: "DFlash 2: Keep
// Drafting Parallel" (inco.ai blog), section "A Lightweight Local Convolution" (two taps, the
// current position and the one before; a learned base kernel plus a correction from the hidden
// state, one correction per 16 channels; the first draft position reads the last verified
// token, row 0 of the block); "DFlash2 Lands in llama.cpp" (ramgpt.org), section "Dynamic Local
// Convolution" (static weight per tap and channel plus a dynamic weight per position, tap and
// channel group; tap by tap with a block-local zero-padded shift; the same dynamic weights on
// both sides of a sublayer, a base kernel per side: one call per side).
//
// Elementwise and HBM-bound: every output is written once and every input read from HBM once. A
// thread owns one 16-byte vector of channels over a segment of kRows rows of one block: it loads
// the segment and the K - 1 rows before it at once (those few extra reads hit the cache the
// neighbouring segment filled), so one memory round trip serves the segment, and a block of
// T rows spreads over ceil(T / kRows) threads per vector (a draft block is short). The
// coefficients of a vector come from its base slice (loaded once) and, per row and tap, the
// dynamic value of its group. Shapes whose rows or groups do not split into 16-byte vectors take
// a one-channel-per-thread kernel. fp32 arithmetic; bf16 outputs are rounded to nearest even.
// The grid is one-dimensional: workgroup index = (block * segments + segment) * column groups +
// column group.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kConvThreads = 256;
// rows loaded ahead per step (fewer with more taps: registers)
constexpr int rows_ahead(int kt) { return kt >= 8 ? 2 : 4; }

template <typename T> struct Out;
template <> struct Out<float> {
    static __device__ __forceinline__ u32x4 pack(const float *v) {
        return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    }
    static __device__ __forceinline__ void store1(float *p, float v) { *p = v; }
};
template <> struct Out<uint16_t> {
    static __device__ __forceinline__ uint32_t pair(float lo, float hi) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 h = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, h);
    }
    static __device__ __forceinline__ u32x4 pack(const float *v) {
        return u32x4{pair(v[0], v[1]), pair(v[2], v[3]), pair(v[4], v[5]), pair(v[6], v[7])};
    }
    static __device__ __forceinline__ void store1(uint16_t *p, float v) {
        *p = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
};

// Vector path: C % EV == 0 (rows stay 16-byte aligned) and G % EV == 0 (a vector lies inside one
// group: one dynamic value per row and tap). KT >= K taps are unrolled.
template <typename T, int KT>
__global__ __launch_bounds__(kConvThreads) __attribute__((amdgpu_waves_per_eu(4))) void
dynconv_vec_kernel(
    const T *__restrict__ x, const T *__restrict__ base, const T *__restrict__ dyn, int Tn, int C,
    int K, int G, T *__restrict__ y) {
    constexpr int EV = Elem<T>::kPerVec;
    constexpr int kRows = rows_ahead(KT);
    const int ncb = (C / EV + kConvThreads - 1) / kConvThreads;  // column groups
    const int nseg = (Tn + kRows - 1) / kRows;
    // (32-bit index arithmetic: a 64-bit division is hundreds of scalar instructions before the
    // first load; the grid's block count fits 32 bits)
    const uint32_t seg_all = blockIdx.x / (uint32_t)ncb;
    const int v = (int)(blockIdx.x % (uint32_t)ncb) * kConvThreads + threadIdx.x;  // channel vector
    const int64_t b = seg_all / (uint32_t)nseg;
    const int t0 = (int)(seg_all % (uint32_t)nseg) * kRows;
    const int c0 = v * EV;
    if (c0 >= C) return;
    const int ng = C / G;
    // base slice and the last KT rows of this vector, kept packed and widened where used
    u32x4 braw[KT], hraw[KT];  // hraw[j]: row t - j
    const T *xb = x + b * Tn * C + c0;
    T *yb = y + b * Tn * C + c0;
    const T *db = dyn + b * Tn * K * ng;
    // the K - 1 rows before the segment (zero before the block start), then the segment
#pragma unroll
    for (int tap = 0; tap < KT; ++tap) {
        braw[tap] = tap < K ? *reinterpret_cast<const u32x4 *>(base + (int64_t)tap * C + c0)
                            : u32x4{0u, 0u, 0u, 0u};
        // row t0 - 1 - tap: the first row's shift moves it to hraw[tap + 1]
        const int tp = t0 - 1 - tap;
        hraw[tap] = tap + 1 < K && tp >= 0
                        ? *reinterpret_cast<const u32x4 *>(xb + (int64_t)tp * C)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 raw[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i)
        raw[i] = t0 + i < Tn ? *reinterpret_cast<const u32x4 *>(xb + (int64_t)(t0 + i) * C)
                             : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int t = t0 + i;
        if (t >= Tn) break;
#pragma unroll
        for (int j = KT - 1; j > 0; --j) hraw[j] = hraw[j - 1];
        hraw[0] = raw[i];
        float out[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e) out[e] = 0.f;
#pragma unroll
        for (int tap = 0; tap < KT; ++tap) {
            if (tap >= K) break;
            float bw[EV], xv[EV];
            Elem<T>::unpack(braw[tap], bw);
            Elem<T>::unpack(hraw[tap], xv);
            const float d = Elem<T>::load(db, ((int64_t)t * K + tap) * ng + c0 / G);
#pragma unroll
            for (int e = 0; e < EV; ++e) out[e] = fmaf(bw[e] + d, xv[e], out[e]);
        }
        *reinterpret_cast<u32x4 *>(yb + (int64_t)t * C) = Out<T>::pack(out);
    }
}

// Any C and group: one channel per thread, scalar loads.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void dynconv_scalar_kernel(
    const T *__restrict__ x, const T *__restrict__ base, const T *__restrict__ dyn, int Tn, int C,
    int K, int G, T *__restrict__ y) {
    const int ncb = (C + kConvThreads - 1) / kConvThreads;
    const int c = (int)(blockIdx.x % ncb) * kConvThreads + threadIdx.x;
    const int64_t b = blockIdx.x / ncb;
    if (c >= C) return;
    const int ng = C / G;
    for (int t = 0; t < Tn; ++t) {
        float out = 0.f;
        for (int tap = 0; tap < K && tap <= t; ++tap) {
            const float w = Elem<T>::load(base, (int64_t)tap * C + c) +
                            Elem<T>::load(dyn, ((b * Tn + t) * K + tap) * ng + c / G);
            out = fmaf(w, Elem<T>::load(x, (b * Tn + t - tap) * C + c), out);
        }
        Out<T>::store1(y + (b * Tn + t) * C + c, out);
    }
}

template <typename T>
hipError_t launch_t(const void *x, const void *base, const void *dyn, int nb, int Tn, int C,
                    int K, int G, void *y, hipStream_t stream) {
    constexpr int EV = Elem<T>::kPerVec;
    const T *xp = static_cast<const T *>(x);
    const T *bp = static_cast<const T *>(base);
    const T *dp = static_cast<const T *>(dyn);
    T *yp = static_cast<T *>(y);
    if (C % EV == 0 && G % EV == 0) {
        auto grid = [&](int kt) {
            const int rows = rows_ahead(kt);
            return dim3((unsigned)((int64_t)((C / EV + kConvThreads - 1) / kConvThreads) * nb *
                                   ((Tn + rows - 1) / rows)));
        };
        if (K <= 2)
            hipLaunchKernelGGL((dynconv_vec_kernel<T, 2>), grid(2), dim3(kConvThreads), 0, stream, xp,
                               bp, dp, Tn, C, K, G, yp);
        else if (K <= 4)
            hipLaunchKernelGGL((dynconv_vec_kernel<T, 4>), grid(4), dim3(kConvThreads), 0, stream, xp,
                               bp, dp, Tn, C, K, G, yp);
        else
            hipLaunchKernelGGL((dynconv_vec_kernel<T, 8>), grid(8), dim3(kConvThreads), 0, stream, xp,
                               bp, dp, Tn, C, K, G, yp);
    } else {
        const dim3 grid((unsigned)((int64_t)((C + kConvThreads - 1) / kConvThreads) * nb));
        hipLaunchKernelGGL((dynconv_scalar_kernel<T>), grid, dim3(kConvThreads), 0, stream, xp, bp,
                           dp, Tn, C, K, G, yp);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dynconv(const void *x, const void *base, const void *dyn, int dtype, int nb,
                          int Tn, int C, int K, int G, void *y, hipStream_t stream) {
    if (dtype == 0) return launch_t<float>(x, base, dyn, nb, Tn, C, K, G, y, stream);
    return launch_t<uint16_t>(x, base, dyn, nb, Tn, C, K, G, y, stream);
}

}  // namespace dflash2
