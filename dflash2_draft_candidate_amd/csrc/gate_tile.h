// The MFMA tile of the gate product g = hidden . W_sel, shared by the stand-alone gate kernel
// and the top-k kernel, which computes one split-K tile per workgroup before it streams.
//
// A wave accumulates a 16-row tile over a range of H in steps of 32 with
// v_mfma_f32_16x16x32_bf16 (fp32 accumulation):
//   * A fragments (8 consecutive h of one row) are 16-byte loads of `hidden`;
//   * W_sel is [H, r] (r contiguous), but a B fragment needs 8 consecutive h of one column. Lane
//     position m loads the NT contiguous columns NT*m .. NT*m + NT - 1 of each of its 8 rows in one
//     vector load (16 lanes cover a row of r = 16 * NT columns: coalesced), and the fragment of
//     tile t takes column NT*m + t from the 8 rows (low halves of the column pairs for even t,
//     high halves for odd t). So the output column of tile t at lane position m is NT*m + t.
//     Every load is independent: a batch of steps is issued before any MFMA runs.
// Sources: "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path
// Selector" (context gate H(h_t)); "DFlash2 Lands in llama.cpp" (ramgpt.org), section "What
// llama.cpp Actually Builds for the Selector" (hidden state through the selector-hidden weight).
#pragma once

#include "device_common.h"

namespace dflash2 {


// Waves sharing one tile's range of H. (Eight waves at 8 column tiles, each with half the
// steps, took as long: the tile costs the stream the same wave-time either way.)
template <int NT> constexpr int gate_waves() { return 4; }
// LDS row pitch (floats) of a wave's part of the tile: padded, except at 16 column tiles (64 KB).
template <int NT> constexpr int gate_pitch() { return NT * 16 + (NT == 16 ? 0 : 1); }
constexpr int kStepK = 32;     // H per MFMA

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// Output column of MFMA tile t at lane position m.
template <int NT>
__device__ __forceinline__ int out_col(int t, int m) {
    return NT * m + t;
}

template <int NT>
struct Step {
    static constexpr int NP = NT == 1 ? 1 : NT / 2;  // column pairs per lane
    u32x4 a;                                        // A fragment
    uint32_t w[8][NP];                              // W rows k0+8g+i, columns NT*m + 2p, +1
};

// Loads of one 32-wide step. FAST (wave-uniform): the step lies inside H, H % 8 == 0 and r is
// exactly the padded tile width (so W_sel rows are 2*NT*16-byte multiples and each lane's
// columns are one aligned vector), so every load is unconditional (rows past R read row R-1 and
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
            if (NT == 1) {
                s.w[i][0] = wrow[m];
            } else {
                typedef uint32_t row_t __attribute__((ext_vector_type(Step<NT>::NP)));
                const row_t v = *reinterpret_cast<const row_t *>(wrow + NT * m);
#pragma unroll
                for (int p = 0; p < Step<NT>::NP; ++p) s.w[i][p] = v[p];
            }
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
                const int c = NT * m + 2 * p;
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
template <int NT> constexpr int batch_steps() { return NT <= 2 ? 4 : (NT == 4 ? 2 : 1); }


// Steps [s0, s1) of wave q of the nq waves that share a tile's H (q = split * 4 + wave). In
// 32 bits: nsteps < 2^26 and q < nq <= 64, so the products fit (a 64-bit division costs hundreds
// of scalar instructions before the wave's first load).
__device__ __forceinline__ void gate_steps(int H, int q, int nq, int &s0, int &s1) {
    const uint32_t nsteps = (uint32_t)(H + kStepK - 1) / kStepK;
    s0 = (int)(nsteps * (uint32_t)q / (uint32_t)nq);
    s1 = (int)(nsteps * (uint32_t)(q + 1) / (uint32_t)nq);
}

// One wave's part of a tile: rows row0 .. row0 + 15 (rows past R read row R - 1 and are dropped
// at the store) over steps [s0, s1). acc[t][i] is row g*4+i, column out_col(t, m) of the tile,
// with m = lane & 15 and g = lane >> 4.
// DB: steps whose loads are issued together; TAIL: a last batch of fewer steps stays on the
// fast path (else it goes step by step). The MFMAs run in step order either way, so every
// choice gives the same sums bit for bit.
template <int NT, int DB = batch_steps<NT>(), bool TAIL = false>
__device__ __forceinline__ void gate_wave(const uint16_t *__restrict__ hidden,
                                          const uint16_t *__restrict__ W, int R, int H, int r,
                                          int row0, int s0, int s1, int lane, f32x4 *acc) {
    constexpr int NC = NT * 16;
    constexpr int D = DB;
    const int m = lane & 15, g = lane >> 4;
    const int row = row0 + m;
    const bool row_ok = row < R;
    const uint16_t *hrow = hidden + (int64_t)(row_ok ? row : 0) * H;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Full batches of D steps on the fast path; everything else (ragged H, odd r) step by step.
    const bool fast_ok = (H % 8) == 0 && r == NC;
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
        if constexpr (TAIL) {
            // the remaining n < D steps that lie inside H, in one batch (uniform conditions)
            const int n = min(s1, H / kStepK) - s;
            if (n > 0) {
                Step<NT> st[D];
#pragma unroll
                for (int d = 0; d < D; ++d)
                    if (d < n) load_step<NT, true>(st[d], hrow, row_ok, W, H, r, (s + d) * kStepK, g, m);
#pragma unroll
                for (int d = 0; d < D; ++d)
                    if (d < n) mma_step<NT>(st[d], acc);
                s += n;
            }
        }
    }
    for (; s < s1; ++s) {
        Step<NT> st;
        load_step<NT, false>(st, hrow, row_ok, W, H, r, s * kStepK, g, m);
        mma_step<NT>(st, acc);
    }
}

}  // namespace dflash2
