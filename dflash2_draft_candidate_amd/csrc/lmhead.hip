// The LM-head product with the top-k pass in its epilogue: the logits never reach HBM.
//
// For each row i of hidden [R, H] and each vocabulary row v of W_lm [V, H] (both bf16; W_lm in
// the usual [vocab, hidden] layout), x_iv = sum_h hidden[i][h] * W_lm[v][h], and the outputs are
// those of the top-k pass over x: the first k tokens of the candidate order (higher logit first,
// equal logits by lower id, +0 == -0), unary_j = x_{cand_j} - logsumexp_v x_iv, and the
// logsumexp. Sources: "DFlash2 Lands in llama.cpp" (ramgpt.org), section "What llama.cpp
// Actually Builds for the Selector" (the per-position top-k is taken over the drafter's logits,
// the output of its full-vocabulary projection, and the walk never reruns that projection) and
// section "The Most Important Performance Question Is Now Different" (top-k candidate extraction
// is one of the draft cycle's costs). Folding the top-k into the projection is this library's
// design: it removes the [R, V] logits round trip through HBM.
//
// Design (gfx950, wave64; four waves per workgroup, no LDS staging of operands; one row tile of
// 16 rows, R <= 16: the decode shape, where W_lm is read once and the pass is bound by that read;
// with more row tiles the weight is reused and a library product with staged tiles is faster):
//   * Work. A workgroup takes the (up to) 16 rows and a contiguous range of the vocabulary;
//     its four waves split the range into contiguous runs of 16-column tiles, and a wave handles
//     its run in passes over H of equal size (at most four tiles). Workgroups number their row blocks XCD by XCD, so the row
//     blocks that read one vocabulary range share its W_lm lines in one L2.
//   * Product. v_mfma_f32_16x16x32_bf16 with fp32 accumulation. Both operands are K-contiguous
//     (rows of hidden for A, rows of W_lm for B): per step of 64 h a lane loads 16 consecutive
//     h of each of its rows (32 bytes; a row's four lane groups read a whole 128-byte line) and
//     feeds them to two MFMAs; four steps of loads are in flight (fewer for larger row tiles).
//     H % 8 == 0; rows past R read row R - 1 and are dropped; tiles past a wave's run issue no
//     loads.
//   * Epilogue. The accumulator of tile (rt, ct) puts row 16 rt + 4 g + t (g = lane / 16) and
//     column 16 ct + (lane % 16) in each lane, so every row lives in one lane group of 16. Each
//     lane keeps an online logsumexp pair (reference = its largest value, log2 domain) per row;
//     each row keeps its 16 best keys (the 64-bit candidate key) sorted across its lane group.
//     A tile's keys are filtered against the larger of the list's 16th key and the smallest of
//     the group's lane maxima (16 of the tile's keys reach it), and the survivors are inserted
//     one per group per step (ballot rank, DPP row shift), all four groups at once.
//   * End. The four waves' lists of each row are sorted together (64 keys) and the best 16 kept;
//     their pairs are combined in wave order. Each workgroup writes [R][ranges] partials, and a
//     second kernel merges a row's ranges (filtered insertion, pairs in range order). The whole
//     path is deterministic.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {


constexpr int kLmWaves = 4;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kLmGroup = 4;            // 16-column tiles per pass of a wave
constexpr int kLmList = 16;            // keys kept per row (>= k)
constexpr int kLmRowTiles = 1;         // 16-row tiles per workgroup (R <= 16)
constexpr int kLmTargetWgs = 512;      // workgroups per launch (about two per CU)
constexpr int kXcds = 8;
constexpr int kDppRowShr1 = 0x111;     // row_shr:1 (within rows of 16 lanes)
constexpr int kDppRowLast = 0x15F;     // row_newbcast:15 (lane 15 of each row to the row)
constexpr int kDppWaveShr1 = 0x138;    // wave_shr:1
constexpr int kDppRowShl4 = 0x104;     // row_shl:4 (lane m reads m + 4)
constexpr int kDppRowShr4 = 0x114;     // row_shr:4 (lane m reads m - 4)
constexpr int kDppRowMirror = 0x140;   // row_mirror (lane m reads 15 - m)
constexpr int kLmFewKeys = 4;          // at most this many new keys per row: insert, else sort

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

// Value of lane src (per-lane index) of v.
__device__ __forceinline__ uint64_t lane_read(uint64_t v, int src) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Wave-uniform value of lane src (src uniform).
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Minimum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ uint32_t row16_min(uint32_t v) {
    v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRor8, 0xF, 0xF, false));
    v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRor4, 0xF, 0xF, false));
    v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, false));
    v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false));
    return v;
}

// Maximum of floats over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ float row16_fmax(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRor8, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRor4, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppXor2, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppXor1, 0xF, 0xF, false)));
    return v;
}

// Lane m ^ s within its row of 16 (s = 1, 2, 4, 8).
template <int S>
__device__ __forceinline__ uint64_t row_xor(uint64_t v, int m) {
    if constexpr (S == 1) {
        return dpp64<kDppXor1>(v);
    } else if constexpr (S == 2) {
        return dpp64<kDppXor2>(v);
    } else if constexpr (S == 8) {
        return dpp64<kDppRor8>(v);
    } else {
        const uint64_t up = dpp64<kDppRowShl4>(v), dn = dpp64<kDppRowShr4>(v);
        return (m & 4) ? dn : up;
    }
}

__device__ __forceinline__ uint64_t row_xor_any(uint64_t v, int s, int m) {
    switch (s) {
    case 1: return row_xor<1>(v, m);
    case 2: return row_xor<2>(v, m);
    case 4: return row_xor<4>(v, m);
    default: return row_xor<8>(v, m);
    }
}

// Bitonic sort of the 64 keys of each lane group (16 lanes x 4 registers; element c * 16 + m is
// register c of lane m of the group) into descending order: register 0 then holds ranks 0..15.
__device__ __forceinline__ void group_sort64(uint64_t *v, int m) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 16) {  // partner: register c ^ (stride / 16) of the same lane
                const int cs = stride / 16;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (c & cs) continue;
                    const bool desc = ((c * 16) & size) == 0;
                    const uint64_t hi = kmax(v[c], v[c | cs]), lo = kmin(v[c], v[c | cs]);
                    v[c] = desc ? hi : lo;
                    v[c | cs] = desc ? lo : hi;
                }
            } else {  // partner: lane m ^ stride, same register
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint64_t o = row_xor_any(v[c], stride, m);
                    const bool desc = ((c * 16 + m) & size) == 0;
                    const bool lower = (m & stride) == 0;
                    v[c] = lower == desc ? kmax(v[c], o) : kmin(v[c], o);
                }
            }
        }
    }
}

// Offer one row slot's keys (kLmGroup columns per lane, 0 = no column) to the row's list. The row
// is this lane's group of 16; lane m of the group holds rank m of the list (descending, 0 =
// empty). tau0: a threshold at or below 16 of the offered keys. When every group has at most
// kLmFewKeys keys above its threshold, each step inserts one key per group (ballot rank, DPP row
// shift); otherwise each group sorts its 64 keys and merges the best 16 into its list (the
// elementwise maximum of the list and the reversed best 16 holds the best 16 of both as a bitonic
// sequence, which four exchange steps sort).
__device__ __forceinline__ void offer_row(uint64_t &list, uint64_t *key, uint64_t tau0, int lane) {
    static_assert(kLmGroup == 4, "the sort network is built for 4 keys per lane");
    const int m = lane & 15, gs = lane & 48;
    uint64_t tau = dpp64<kDppRowLast>(list);
    const uint64_t lim = tau > tau0 ? tau : tau0;
    uint64_t pend[kLmGroup];
#pragma unroll
    for (int c = 0; c < kLmGroup; ++c) pend[c] = __ballot(key[c] != 0ull && key[c] >= lim);
    uint32_t n = 0;  // this lane's group: pending keys
#pragma unroll
    for (int c = 0; c < kLmGroup; ++c) n += (uint32_t)__popc((uint32_t)(pend[c] >> gs) & 0xFFFFu);
    if (__ballot(n > kLmFewKeys) != 0ull) {
        group_sort64(key, m);
        uint64_t x = kmax(list, dpp64<kDppRowMirror>(key[0]));
#pragma unroll
        for (int stride = 8; stride > 0; stride >>= 1) {
            const uint64_t o = row_xor_any(x, stride, m);
            x = (m & stride) == 0 ? kmax(x, o) : kmin(x, o);
        }
        list = x;
        return;
    }
    for (;;) {
        int sel = -1, sm = 0;
#pragma unroll
        for (int c = kLmGroup - 1; c >= 0; --c) {
            const uint32_t gp = (uint32_t)(pend[c] >> gs) & 0xFFFFu;
            if (gp) {
                sel = c;
                sm = __builtin_ctz(gp);
            }
        }
        if (__ballot(sel >= 0) == 0ull) break;
        uint64_t kv = key[0];
#pragma unroll
        for (int c = 1; c < kLmGroup; ++c) kv = sel == c ? key[c] : kv;
        const uint64_t cand = lane_read(kv, gs + sm);
#pragma unroll
        for (int c = 0; c < kLmGroup; ++c) pend[c] &= ~__ballot(sel == c && m == sm);
        const bool ins = sel >= 0 && cand > tau;
        const int rank = __popc((uint32_t)(__ballot(list > cand) >> gs) & 0xFFFFu);
        const uint64_t shifted = dpp64<kDppRowShr1>(list);
        if (ins) list = m < rank ? list : (m == rank ? cand : shifted);
        tau = dpp64<kDppRowLast>(list);
    }
}

struct LmJob {
    const uint16_t *hidden;  // [R, H]
    const uint16_t *W;       // [V, H]
    int R, H, V;
    int rblocks;             // row blocks of 16 * RT rows (one)
    int ranges;              // vocabulary ranges (workgroups per row block)
    int col16;               // 16-column tiles in V
    uint64_t *part_keys;     // [R][ranges][kLmList]
    float2 *part_lse;        // [R][ranges] (log2-domain reference, sum)
};

// Workgroup (row block, range): the row block of one range on one XCD (see the header).
__global__ __launch_bounds__(kLmThreads) void lmhead_topk_kernel(LmJob job) {
    constexpr int RT = kLmRowTiles;
    constexpr int D = 4;  // steps of loads in flight
    __shared__ uint64_t lists[kLmWaves][16 * RT][16];
    __shared__ float2 pairs[kLmWaves][16 * RT];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 15, g = lane >> 4;
    const int n = (int)gridDim.x;
    const int t = n % kXcds == 0 ? ((int)blockIdx.x % kXcds) * (n / kXcds) + (int)blockIdx.x / kXcds
                                 : (int)blockIdx.x;
    const int rb = t % job.rblocks, range = t / job.rblocks;
    const int H = job.H, V = job.V;
    const int row0 = rb * 16 * RT;
    const int nw = job.ranges * kLmWaves, gw = range * kLmWaves + wave;
    const int tc0 = (int)((int64_t)job.col16 * gw / nw), tc1 = (int)((int64_t)job.col16 * (gw + 1) / nw);

    const uint16_t *arow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        arow[rt] = job.hidden + (int64_t)min(row0 + 16 * rt + m, job.R - 1) * H;

    uint64_t list[RT][4];
    float lref[RT][4], lsum[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            list[rt][i] = 0ull;
            lref[rt][i] = -INFINITY;
            lsum[rt][i] = 0.f;
        }

    const int ns = (H + 63) / 64;  // steps over H (two MFMAs each)
    // passes of equal size (at most kLmGroup tiles): no pass much smaller than the others
    const int npass = (tc1 - tc0 + kLmGroup - 1) / kLmGroup;
    const int per = npass > 0 ? (tc1 - tc0 + npass - 1) / npass : kLmGroup;
    for (int tc = tc0; tc < tc1; tc += per) {
        const int te = min(tc + per, tc1);  // this pass: tiles tc .. te - 1
        const uint16_t *brow[kLmGroup];
#pragma unroll
        for (int c = 0; c < kLmGroup; ++c)
            brow[c] = job.W + (int64_t)min((tc + c) * 16 + m, V - 1) * H;
        f32x4 acc[RT][kLmGroup];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int c = 0; c < kLmGroup; ++c) acc[rt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        // A step covers 64 of H: lane group g loads the 16 consecutive h at 64 s + 16 g of each
        // row (32 bytes: four groups cover a 128-byte line), and the two MFMAs of the step take
        // the first and the second 8 as their K slots 8 g .. 8 g + 7 (the same map for both
        // operands, so the sum over h is unchanged). Tiles past the wave's run load nothing.
        const int live = te - tc;
        u32x4 fa[D][RT][2], fb[D][kLmGroup][2];
        auto load = [&](int d, int s) {
            const int kc = 64 * s + 16 * g;
            const bool ok0 = kc < H, ok1 = kc + 8 < H;  // H % 8 == 0
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                fa[d][rt][0] = ok0 ? *reinterpret_cast<const u32x4 *>(arow[rt] + kc) : u32x4{0u, 0u, 0u, 0u};
                fa[d][rt][1] = ok1 ? *reinterpret_cast<const u32x4 *>(arow[rt] + kc + 8) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int c = 0; c < kLmGroup; ++c) {
                const bool on = c < live;
                fb[d][c][0] = on && ok0 ? *reinterpret_cast<const u32x4 *>(brow[c] + kc) : u32x4{0u, 0u, 0u, 0u};
                fb[d][c][1] = on && ok1 ? *reinterpret_cast<const u32x4 *>(brow[c] + kc + 8) : u32x4{0u, 0u, 0u, 0u};
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (d < ns) load(d, d);
        for (int s0 = 0; s0 < ns; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int s = s0 + d;
                if (s < ns) {
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                            for (int c = 0; c < kLmGroup; ++c)
                                acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, fa[d][rt][hf]),
                                    __builtin_bit_cast(bf16x8, fb[d][c][hf]), acc[rt][c], 0, 0, 0);
                    if (s + D < ns) load(d, s + D);
                }
            }
        }

        // Epilogue: row 16 rt + 4 g + i, column (tc + c) * 16 + m.
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint64_t key[kLmGroup];
                float xl[kLmGroup];
                float xm = -INFINITY;
                uint32_t vmax = 0u;
#pragma unroll
                for (int c = 0; c < kLmGroup; ++c) {
                    const int col = (tc + c) * 16 + m;
                    const bool ok = tc + c < te && col < V;
                    const float x = acc[rt][c][i];
                    key[c] = ok ? cand_key(x, col) : 0ull;
                    xl[c] = ok ? x * kLog2e : -INFINITY;
                    xm = fmaxf(xm, xl[c]);
                    vmax = ok && (uint32_t)(key[c] >> 32) > vmax ? (uint32_t)(key[c] >> 32) : vmax;
                }
                if (xm != -INFINITY) {
                    if (xm > lref[rt][i]) {
                        lsum[rt][i] *= __builtin_amdgcn_exp2f(lref[rt][i] - xm);
                        lref[rt][i] = xm;
                    }
                    float s = 0.f;
#pragma unroll
                    for (int c = 0; c < kLmGroup; ++c)
                        s += xl[c] != -INFINITY ? __builtin_amdgcn_exp2f(xl[c] - lref[rt][i]) : 0.f;
                    lsum[rt][i] += s;
                }
                const uint64_t tau0 = (uint64_t)row16_min(vmax) << 32;
                offer_row(list[rt][i], key, tau0, lane);
            }
        }
    }

    // The wave's lists and pairs to LDS; then each row's four lists are sorted together.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 16 * rt + 4 * g + i;
            lists[wave][rl][m] = list[rt][i];
            const float ref = row16_fmax(lref[rt][i]);
            float s = ref == -INFINITY ? 0.f : lsum[rt][i] * __builtin_amdgcn_exp2f(lref[rt][i] - ref);
            s = row16_sum(s);
            if (m == 0) pairs[wave][rl] = make_float2(ref, s);
        }
    }
    __syncthreads();
    for (int rl = wave; rl < 16 * RT; rl += kLmWaves) {
        const int row = row0 + rl;
        if (row >= job.R) break;
        uint64_t key = lists[lane >> 4][rl][lane & 15];
        key = wave_sort_desc(key, lane);
        const size_t part = (size_t)row * job.ranges + range;
        if (lane < kLmList) job.part_keys[part * kLmList + lane] = key;
        if (lane == 0) {
            float ref = -INFINITY, sum = 0.f;
#pragma unroll
            for (int w = 0; w < kLmWaves; ++w) lse_combine(ref, sum, pairs[w][rl].x, pairs[w][rl].y);
            job.part_lse[part] = make_float2(ref, sum);
        }
    }
}

// One workgroup of kMergeWaves waves per row; the row's ranges are each sorted lists of kLmList
// keys. Wave w takes ranges [w, w + 1) * ranges / 16 (at most 32, as ranges <= kLmTargetWgs)
// and loads all their keys at once (lane j holds key j % 16 of ranges r0 + j / 16 + 4 s, s < 8:
// one memory round trip). A threshold T: the k-th largest of the ranges' first (largest) keys,
// which are distinct real keys, so the top k of the row are all >= T; and only the ranges whose
// first key is >= T hold keys >= T. Wave 0 finds T (below) such that at most 64 ranges reach it,
// so at most kLmList * 64 keys pass; they go to LDS, and wave 0 sorts them (64 at a time,
// merged) and keeps the top k. The (ref, sum) pairs are combined per wave by a fixed shuffle
// tree, then over the waves in order.
constexpr int kMergeWaves = 16;
constexpr int kMergeSteps = 8;  // 4 ranges per step: 32 ranges per wave
static_assert(kMergeWaves * (kWave / kLmList) * kMergeSteps >= kLmTargetWgs,
              "every range of a row has a load slot");
constexpr int kMergeCands = kLmList * kWave;  // keys >= T at most

// The k-th largest of the 64 lane values (one per lane, 0 = none, nonzero ones distinct): the
// largest t with at least k lane values >= t, one bit at a time from the top.
__device__ __forceinline__ uint64_t kth_largest(uint64_t v, int k) {
    uint64_t t = 0ull;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t c = t | (1ull << bit);
        if (__popcll(__ballot(v >= c)) >= k) t = c;
    }
    return t;
}

// A threshold for the n <= 512 distinct first keys in LDS (zeros elsewhere), by one wave: the
// k-th largest T1 of the 64 lane-wise maxima (k distinct firsts reach it, so every key of the
// row's top k is >= T1) when at most 64 firsts reach it (the usual case), else the k-th largest
// of all firsts (exactly k reach it).
__device__ __forceinline__ uint64_t merge_threshold(const uint64_t *firsts, int k, int lane) {
    constexpr int J = kLmTargetWgs / kWave;
    uint64_t f[J], m = 0ull;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        f[j] = firsts[lane + kWave * j];
        m = kmax(m, f[j]);
    }
    const uint64_t t1 = kth_largest(m, k);
    uint32_t n1 = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j) n1 += (uint32_t)__popcll(__ballot(f[j] != 0ull && f[j] >= t1));
    if (n1 > (uint32_t)kWave) {  // many firsts at or above T1: count all of them per bit
        uint64_t t = 0ull;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t c = t | (1ull << bit);
            int n = 0;
#pragma unroll
            for (int j = 0; j < J; ++j) n += __popcll(__ballot(f[j] >= c));
            if (n >= k) t = c;
        }
        return t;
    }
    return t1;
}

__global__ __launch_bounds__(kMergeWaves * kWave) void lmhead_merge_kernel(
    const uint64_t *__restrict__ part_keys, const float2 *__restrict__ part_lse, int ranges, int k,
    int32_t *__restrict__ cand_ids, float *__restrict__ unary, float *__restrict__ lse_out) {
    __shared__ uint64_t firsts[kLmTargetWgs];   // each range's largest key (0: no range)
    __shared__ uint64_t cands[kMergeCands];
    __shared__ uint32_t ncand;
    __shared__ uint64_t thr;
    __shared__ float2 wp[kMergeWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = blockIdx.x;
    const int r0 = ranges * wave / kMergeWaves, r1 = ranges * (wave + 1) / kMergeWaves;
    constexpr int kPer = kWave / kLmList;  // ranges per step
    uint64_t key[kMergeSteps];
#pragma unroll
    for (int st = 0; st < kMergeSteps; ++st) {
        const int rr = r0 + lane / kLmList + kPer * st;
        key[st] = rr < r1 ? part_keys[((size_t)row * ranges + rr) * kLmList + (lane % kLmList)]
                          : 0ull;
    }
    const float2 pr = r0 + lane < r1 ? part_lse[(size_t)row * ranges + r0 + lane]
                                     : make_float2(-INFINITY, 0.f);
    if (threadIdx.x == 0) ncand = 0u;
    for (int i = threadIdx.x; i < kLmTargetWgs; i += kMergeWaves * kWave) firsts[i] = 0ull;
    {  // (ref, sum) of the wave's ranges: lanes 0 .. r1 - r0 - 1, combined by a fixed tree
        float ref = pr.x, sum = pr.y;
#pragma unroll
        for (int d = 1; d < kWave / 2; d *= 2) {
            const float oref = __shfl_down(ref, d, kWave), osum = __shfl_down(sum, d, kWave);
            if (lane % (2 * d) == 0) lse_combine(ref, sum, oref, osum);
        }
        if (lane == 0) wp[wave] = make_float2(ref, sum);
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < kMergeSteps; ++st) {
        const int rr = r0 + lane / kLmList + kPer * st;
        if (lane % kLmList == 0 && rr < r1) firsts[rr] = key[st];
    }
    __syncthreads();
    if (wave == 0) {
        const uint64_t t = merge_threshold(firsts, k, lane);
        if (lane == 0) thr = t;
    }
    __syncthreads();
    const uint64_t T = thr;
    // the keys >= T to LDS
#pragma unroll
    for (int st = 0; st < kMergeSteps; ++st) {
        const bool pass = key[st] != 0ull && key[st] >= T;
        const uint64_t m = __ballot(pass);
        if (m == 0ull) continue;
        uint32_t base = 0u;
        if (lane == 0)
            base = __hip_atomic_fetch_add(&ncand, (uint32_t)__popcll(m), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP);
        base = __builtin_amdgcn_readfirstlane(base);
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (pass) cands[base + rank] = key[st];
    }
    __syncthreads();
    if (wave != 0) return;
    const uint32_t n = __builtin_amdgcn_readfirstlane(ncand);
    uint64_t top = 0ull;
    for (uint32_t c0 = 0; c0 < n; c0 += kWave) {
        const uint64_t c = c0 + lane < n ? cands[c0 + lane] : 0ull;
        top = wave_merge_desc(top, wave_sort_desc(c, lane), lane);
    }
    float ref = -INFINITY, sum = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) lse_combine(ref, sum, wp[w].x, wp[w].y);
    const double lse = lse_value(ref, sum);
    if (lane < k) {
        cand_ids[row * k + lane] = key_id(top);
        unary[row * k + lane] = (float)((double)key_logit(top) - lse);
    }
    if (lane == 0 && lse_out) lse_out[row] = (float)lse;
}

struct LmPlan {
    int rblocks, ranges, col16;
};

LmPlan plan_lmhead(int R, int V) {
    LmPlan p;
    p.rblocks = (R + 16 * kLmRowTiles - 1) / (16 * kLmRowTiles);
    p.col16 = (V + 15) / 16;
    int ranges = kLmTargetWgs / p.rblocks;
    if (ranges < 1) ranges = 1;
    const int most = (p.col16 + kLmWaves - 1) / kLmWaves;  // every wave gets a tile
    p.ranges = ranges < most ? ranges : most;
    return p;
}

}  // namespace

int lmhead_max_k() { return kLmList; }

size_t lmhead_workspace_bytes(int R, int V) {
    const LmPlan p = plan_lmhead(R, V);
    return (size_t)R * p.ranges * (kLmList * sizeof(uint64_t) + sizeof(float2));
}

hipError_t launch_lmhead_topk(const void *hidden, const void *W_lm, int R, int H, int V, int k,
                              int32_t *cand_ids, float *unary, float *lse, void *workspace,
                              hipStream_t stream) {
    const LmPlan p = plan_lmhead(R, V);
    LmJob job;
    job.hidden = static_cast<const uint16_t *>(hidden);
    job.W = static_cast<const uint16_t *>(W_lm);
    job.R = R;
    job.H = H;
    job.V = V;
    job.rblocks = p.rblocks;
    job.ranges = p.ranges;
    job.col16 = p.col16;
    job.part_keys = static_cast<uint64_t *>(workspace);
    job.part_lse = reinterpret_cast<float2 *>(job.part_keys + (size_t)R * p.ranges * kLmList);
    if (R > 16 * kLmRowTiles) return hipErrorInvalidValue;  // the C ABI refuses these sizes
    hipLaunchKernelGGL(lmhead_topk_kernel, dim3((unsigned)(job.rblocks * job.ranges)),
                       dim3(kLmThreads), 0, stream, job);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3((unsigned)R), dim3(kMergeWaves * kWave), 0, stream,
                       job.part_keys, job.part_lse, p.ranges, k, cand_ids, unary, lse);
    return hipGetLastError();
}

}  // namespace dflash2
