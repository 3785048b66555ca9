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
// Design (gfx950, wave64; one workgroup of eight waves per CU, R <= 16: the decode shape, where
// W_lm is read once and the pass is bound by that read):
//   * Work. A workgroup takes the (up to) 16 rows and a contiguous range of 16-column tiles of
//     the vocabulary; a tile is 16 rows of W_lm, 16 H contiguous values. Wave w owns the 512-h
//     chunks w, w + 8, ... of every tile of the range, so for H <= 4096 each wave holds the
//     hidden rows' fragments of its chunk in registers for the whole pass (for a larger H a
//     wave reloads them, from L2, for each of its chunks).
//   * Stream. Per tile a wave reads, for each of the 16 rows, the row's 1 KB run of its chunk
//     with one 16-byte nontemporal buffer load per lane (the eight waves together read each row
//     whole); the next tile's loads are in flight while the current one is multiplied. Loads
//     that cover 1 KB of one row each ran at 0.80 of the HBM peak on this access order; loads
//     that cover 64 bytes of each of 16 rows (the layout an MFMA fragment wants) at 0.69.
//   * Product. The wave writes its 16 runs to its own LDS area (rows padded by 16 bytes, so the
//     reads below are free of bank conflicts) and reads them back as MFMA fragments: lane (n, kg)
//     takes row n at h = 32 s + 8 kg of the chunk for k-slice s. v_mfma_f32_16x16x32_bf16 with
//     fp32 accumulation over the chunk's 16 k-slices (K slot 8 kg + e is h = 32 s + 8 kg + e for
//     both operands); h past H is zero on both sides.
//   * Reduction. Each wave leaves its partial 16 x 16 tile in LDS (two buffers, one barrier per
//     tile); wave i < 4 adds the waves' partials of rows 4 g + i (g < 4) in wave order and runs
//     their epilogue, so four waves share it.
//   * Epilogue (waves 0..3). The accumulator layout puts row 4 g + i (g = lane / 16, i < 4) and
//     column lane % 16 in each lane, so every row lives in one lane group of 16. Each lane keeps an
//     online logsumexp pair (reference = its largest value, log2 domain) per row; each row keeps
//     its 16 best keys (the 64-bit candidate key) sorted across its lane group. Every four tiles
//     the keys are filtered against the larger of the list's 16th key and the smallest of the
//     group's lane maxima (16 of the offered keys reach it), and the survivors are inserted one
//     per group per step (ballot rank, DPP row shift), or, when a group has more than four, sorted
//     and merged.
//   * End. Each workgroup writes [R][ranges] partials (a sorted list of 16 keys and a pair per
//     row), and a second kernel merges a row's ranges. The whole path is deterministic.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {


constexpr int kLmWaves = 8;            // waves per workgroup
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kLmChunk = 512;          // h per chunk: a 1 KB run of each weight row
constexpr int kLmSlices = kLmChunk / 32;  // k-slices (MFMAs) per chunk
constexpr int kLmRowSlots = kLmChunk / 8 + 1;  // 16-byte slots per staged row, one of padding
constexpr int kLmGroup = 4;            // tiles whose keys the epilogue offers at once
constexpr int kLmList = 16;            // keys kept per row (>= k)
constexpr int kLmWgs = 256;            // workgroups per launch (the LDS holds one per CU)
constexpr int kLmMaxRanges = 512;      // ranges per row the merge kernel takes at most
constexpr int kBufWord3 = 0x00020000;  // gfx9-family buffer descriptor word 3 (raw data)
constexpr int kNonTemp = 2;            // cache policy: streaming data, read once
constexpr int kDppRowShr1 = 0x111;     // row_shr:1 (within rows of 16 lanes)
constexpr int kDppRowLast = 0x15F;     // row_newbcast:15 (lane 15 of each row to the row)
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
    int ranges;              // vocabulary ranges (one workgroup each)
    int col16;               // 16-column tiles in V
    uint64_t *part_keys;     // [R][ranges][kLmList]
    float2 *part_lse;        // [R][ranges] (log2-domain reference, sum)
};

// The hidden rows' MFMA fragments of chunk c: for k-slice s, lane (i, kg) holds h = 512 c + 32 s
// + 8 kg .. + 7 of row i (zero past H and for rows past R).
__device__ __forceinline__ void load_hidden_chunk(const LmJob &job, int c, int lane,
                                                  u32x4 (&a)[kLmSlices]) {
    const int i = lane & 15, kg = lane >> 4;
    const bool row_ok = i < job.R;
    const uint16_t *ar = job.hidden + (int64_t)(row_ok ? i : 0) * job.H;
#pragma unroll
    for (int s = 0; s < kLmSlices; ++s) {
        const int h = kLmChunk * c + 32 * s + 8 * kg;
        a[s] = row_ok && h < job.H ? *reinterpret_cast<const u32x4 *>(ar + h) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Workgroup = one vocabulary range (see the header).
__global__ __launch_bounds__(kLmThreads) void lmhead_topk_kernel(LmJob job) {
    __shared__ u32x4 stage[kLmWaves][16][kLmRowSlots];  // each wave's chunk of the current tile
    __shared__ f32x4 part[2][kLmWaves][kWave];          // the waves' partial tiles (two tiles)

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 15, g = lane >> 4;
    const int H = job.H, V = job.V;
    const int range = blockIdx.x;
    const int t0 = (int)((int64_t)job.col16 * range / job.ranges);
    const int nt = (int)((int64_t)job.col16 * (range + 1) / job.ranges) - t0;
    const int nc = (H + kLmChunk - 1) / kLmChunk;                          // chunks per tile
    const int cpw = wave < nc ? (nc - 1 - wave) / kLmWaves + 1 : 0;        // this wave's
    const int nwv = nc < kLmWaves ? nc : kLmWaves;                         // waves with a chunk

    // (with one chunk per wave they stay for the whole pass; with more, each chunk reloads them)
    u32x4 afr[kLmSlices];
    if (cpw == 1) load_hidden_chunk(job, wave, lane, afr);

    // Loads of chunk wave + 8 j of tile t0 + ti: stg[r] = row r's 16 bytes at h = 512 c + 8 lane
    // (zero past H, and for rows past V: the descriptor ends at the last row).
    u32x4 stg[16];
    auto issue = [&](int ti, int j) {
        const int tile = t0 + ti, c = wave + kLmWaves * j;
        const int rows = min(16, V - tile * 16);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(job.W + (int64_t)tile * 16 * H), (short)0, rows * H * 2, kBufWord3);
        const int h = kLmChunk * c + 8 * lane;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            stg[r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, h < H ? (r * H + h) * 2 : 0x7FFFFFF0,
                                                             0, kNonTemp));
    };
    if (cpw > 0 && nt > 0) issue(0, 0);

    // Epilogue waves 0..3: wave i keeps row 4 g + i of the tile in lane group g.
    const int ei = wave;  // (rows only for ei < 4)
    uint64_t list = 0ull;
    float lref = -INFINITY, lsum = 0.f, xs[kLmGroup];
#pragma unroll
    for (int c = 0; c < kLmGroup; ++c) xs[c] = 0.f;

    for (int ti = 0; ti < nt; ++ti) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < cpw; ++j) {
            // the chunk's rows to the wave's area, the next chunk's loads, then the MFMAs over
            // the fragments read back (same wave: LDS operations complete in order)
#pragma unroll
            for (int r = 0; r < 16; ++r) stage[wave][r][lane] = stg[r];
            if (j + 1 < cpw) issue(ti, j + 1);
            else if (ti + 1 < nt) issue(ti + 1, 0);
            if (cpw > 1) load_hidden_chunk(job, wave + kLmWaves * j, lane, afr);
#pragma unroll
            for (int s = 0; s < kLmSlices; ++s) {
                const u32x4 b = stage[wave][m][4 * s + g];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, afr[s]),
                                                              __builtin_bit_cast(bf16x8, b), acc, 0,
                                                              0, 0);
            }
        }
        if (cpw > 0) part[ti & 1][wave][lane] = acc;
        __syncthreads();
        if (ei >= 4) continue;

        // Epilogue: row 4 g + ei of the tile's logits (the waves' partials added in wave order),
        // kept for a group of tiles.
        const float *pp = reinterpret_cast<const float *>(&part[ti & 1][0][lane]) + ei;
        float x = pp[0];
        for (int w = 1; w < nwv; ++w) x += pp[w * kWave * 4];
        const int slot = ti % kLmGroup;
#pragma unroll
        for (int c = 0; c < kLmGroup; ++c) xs[c] = slot == c ? x : xs[c];
        if (slot != kLmGroup - 1 && ti != nt - 1) continue;
        // column (tb + c) * 16 + m for the group's tiles c <= slot
        const int tb = t0 + ti - slot;
        uint64_t key[kLmGroup];
        float xl[kLmGroup];
        float xm = -INFINITY;
        uint32_t vmax = 0u;
#pragma unroll
        for (int c = 0; c < kLmGroup; ++c) {
            const int col = (tb + c) * 16 + m;
            const bool ok = c <= slot && col < V;
            key[c] = ok ? cand_key(xs[c], col) : 0ull;
            xl[c] = ok ? xs[c] * kLog2e : -INFINITY;
            xm = fmaxf(xm, xl[c]);
            vmax = ok && (uint32_t)(key[c] >> 32) > vmax ? (uint32_t)(key[c] >> 32) : vmax;
        }
        if (xm != -INFINITY) {
            if (xm > lref) {
                lsum *= __builtin_amdgcn_exp2f(lref - xm);
                lref = xm;
            }
            float sacc = 0.f;
#pragma unroll
            for (int c = 0; c < kLmGroup; ++c)
                sacc += xl[c] != -INFINITY ? __builtin_amdgcn_exp2f(xl[c] - lref) : 0.f;
            lsum += sacc;
        }
        const uint64_t tau0 = (uint64_t)row16_min(vmax) << 32;
        offer_row(list, key, tau0, lane);
    }

    // waves 0..3: each row's list (ranks in lane order) and pair to the range's partial
    if (ei >= 4) return;
    const int row = 4 * g + ei;
    const float ref = row16_fmax(lref);
    float sm = ref == -INFINITY ? 0.f : lsum * __builtin_amdgcn_exp2f(lref - ref);
    sm = row16_sum(sm);
    if (row < job.R) {
        const size_t pi = (size_t)row * job.ranges + range;
        job.part_keys[pi * kLmList + m] = list;
        if (m == 0) job.part_lse[pi] = make_float2(ref, sm);
    }
}

// One workgroup of kMergeWaves waves per row; the row's ranges are each sorted lists of kLmList
// keys. Wave w takes ranges [w, w + 1) * ranges / 16 (at most 32, as ranges <= kLmMaxRanges)
// and loads all their keys at once (lane j holds key j % 16 of ranges r0 + j / 16 + 4 s, s < 8:
// one memory round trip). A threshold T: the k-th largest of the ranges' first (largest) keys,
// which are distinct real keys, so the top k of the row are all >= T; and only the ranges whose
// first key is >= T hold keys >= T. Wave 0 finds T (below) such that at most 64 ranges reach it,
// so at most kLmList * 64 keys pass; they go to LDS, and wave 0 sorts them (64 at a time,
// merged) and keeps the top k. The (ref, sum) pairs are combined per wave by a fixed shuffle
// tree, then over the waves in order.
constexpr int kMergeWaves = 16;
constexpr int kMergeSteps = 8;  // 4 ranges per step: 32 ranges per wave
static_assert(kMergeWaves * (kWave / kLmList) * kMergeSteps >= kLmMaxRanges,
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
    constexpr int J = kLmMaxRanges / kWave;
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
    __shared__ uint64_t firsts[kLmMaxRanges];   // each range's largest key (0: no range)
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
    for (int i = threadIdx.x; i < kLmMaxRanges; i += kMergeWaves * kWave) firsts[i] = 0ull;
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
    int ranges, col16;
};

LmPlan plan_lmhead(int R, int V) {
    (void)R;
    LmPlan p;
    p.col16 = (V + 15) / 16;
    p.ranges = p.col16 < kLmWgs ? p.col16 : kLmWgs;  // every workgroup gets a tile
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
    job.ranges = p.ranges;
    job.col16 = p.col16;
    job.part_keys = static_cast<uint64_t *>(workspace);
    job.part_lse = reinterpret_cast<float2 *>(job.part_keys + (size_t)R * p.ranges * kLmList);
    if (R > 16) return hipErrorInvalidValue;  // the C ABI refuses these sizes
    hipLaunchKernelGGL(lmhead_topk_kernel, dim3((unsigned)job.ranges), dim3(kLmThreads), 0, stream,
                       job);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3((unsigned)R), dim3(kMergeWaves * kWave), 0, stream,
                       job.part_keys, job.part_lse, p.ranges, k, cand_ids, unary, lse);
    return hipGetLastError();
}

}  // namespace dflash2
