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
//     their epilogue, so four waves share it. A tile's epilogue runs during the next tile's
//     iteration, after that iteration's loads are issued, so it overlaps their memory latency.
//   * Epilogue (waves 0..3). The accumulator layout puts row 4 g + i (g = lane / 16, i < 4) and
//     column lane % 16 in each lane, so every row lives in one lane group of 16. Each lane keeps an
//     online logsumexp pair (reference = its largest value, log2 domain) per row; each row keeps
//     its 16 best keys (the 64-bit candidate key) sorted across its lane group. Every four tiles
//     the keys are filtered against the larger of the list's 16th key and the smallest of the
//     group's lane maxima (16 of the offered keys reach it), and the survivors are inserted one
//     per group per step (ballot rank, DPP row shift), or, when a group has more than four, sorted
//     and merged.
//   * End. Each workgroup writes [R][ranges] partials (a sorted list of 16 keys and a pair per
//     row), and a second kernel merges each row's ranges with one wave. The whole path is
//     deterministic.
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
    int k;
    uint64_t *part_keys;     // [R][ranges][kLmList]
    float2 *part_lse;        // [R][ranges] (log2-domain reference, sum)
    int32_t *cand_ids;       // [R, k]
    float *unary;            // [R, k]
    float *lse_out;          // [R] or null
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
        a[s] = row_ok && h < job.H ? *reinterpret_cast<const u32x4 *>(ar + h)
                                   : u32x4{0u, 0u, 0u, 0u};
    }
}

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

constexpr int kLmRangesPerLane = kLmWgs / kWave;  // ranges a lane reads in the merge
constexpr int kLmPoolKeys = kWave * kLmList;      // keys >= T at most (64 ranges' lists)

// Row `row`'s merge by one wave: the ranges are each sorted lists of kLmList keys. T: the k-th
// largest of the 64 lane-wise maxima of the ranges' first (largest) keys, which are distinct real
// keys, so k of them reach T and every key of the row's first k is >= T; only ranges whose first
// key reaches T hold such keys. When more than 64 firsts reach T, T becomes the exact k-th
// largest first (then exactly k do). The chosen ranges' keys >= T go to LDS and are sorted 64 at
// a time and merged. The ranges' pairs are combined per lane in range order, then by a fixed
// lane tree. (pool: kLmPoolKeys keys, then 64 range indices.) Two dependent load rounds, no
// barrier.
__device__ __forceinline__ void merge_row(const LmJob &job, int row, uint64_t *pool, int lane) {
    constexpr int Q = kLmRangesPerLane;
    const int nr = job.ranges, k = job.k;
    const uint64_t *pk = job.part_keys + (size_t)row * nr * kLmList;
    const uint64_t *pl = reinterpret_cast<const uint64_t *>(job.part_lse + (size_t)row * nr);
    uint64_t f[Q], pp[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int r = lane + kWave * q;
        f[q] = r < nr ? pk[(size_t)r * kLmList] : 0ull;
        pp[q] = r < nr ? pl[r] : 0ull;
    }
    float ref = -INFINITY, sum = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (lane + kWave * q < nr)
            lse_combine(ref, sum, __uint_as_float((uint32_t)pp[q]),
                        __uint_as_float((uint32_t)(pp[q] >> 32)));
#pragma unroll
    for (int d = 1; d < kWave; d *= 2) {
        const float oref = __shfl_down(ref, d, kWave), osum = __shfl_down(sum, d, kWave);
        if (lane % (2 * d) == 0) lse_combine(ref, sum, oref, osum);
    }
    ref = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(ref)));
    sum = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(sum)));

    uint64_t mx = f[0];
#pragma unroll
    for (int q = 1; q < Q; ++q) mx = kmax(mx, f[q]);
    uint64_t T = kth_largest(mx, k);
    uint32_t n1 = 0u;
#pragma unroll
    for (int q = 0; q < Q; ++q) n1 += (uint32_t)__popcll(__ballot(f[q] != 0ull && f[q] >= T));
    if (n1 > (uint32_t)kWave) {  // many firsts at or above T: the exact k-th largest first
        uint64_t t = 0ull;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t c = t | (1ull << bit);
            int n = 0;
#pragma unroll
            for (int q = 0; q < Q; ++q) n += __popcll(__ballot(f[q] >= c));
            if (n >= k) t = c;
        }
        T = t;
    }
    // the chosen ranges' indices (at most 64), then their keys >= T
    uint32_t *idx = reinterpret_cast<uint32_t *>(pool + kLmPoolKeys);
    uint32_t nsel = 0u;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const bool in = f[q] != 0ull && f[q] >= T;
        const uint64_t m = __ballot(in);
        if (in)
            idx[nsel + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
                (uint32_t)(lane + kWave * q);
        nsel += (uint32_t)__popcll(m);
    }
    const bool have = (uint32_t)lane < nsel;
    const uint32_t rr = have ? idx[lane] : 0u;
    uint64_t kk[kLmList];
#pragma unroll
    for (int i = 0; i < kLmList; ++i)
        kk[i] = have ? pk[(size_t)rr * kLmList + i] : 0ull;
    uint32_t n = 0u;
#pragma unroll
    for (int i = 0; i < kLmList; ++i) {
        const bool in = kk[i] != 0ull && kk[i] >= T;
        const uint64_t m = __ballot(in);
        if (in)
            pool[n + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = kk[i];
        n += (uint32_t)__popcll(m);
    }
    uint64_t top = 0ull;
    for (uint32_t c0 = 0; c0 < n; c0 += kWave) {
        const uint64_t c = c0 + lane < n ? pool[c0 + lane] : 0ull;
        top = wave_merge_desc(top, wave_sort_desc(c, lane), lane);
    }
    const double lse = lse_value(ref, sum);
    if (lane < k) {
        job.cand_ids[row * k + lane] = key_id(top);
        job.unary[row * k + lane] = (float)((double)key_logit(top) - lse);
    }
    if (lane == 0 && job.lse_out) job.lse_out[row] = (float)lse;
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
    // the range's 16-column tiles [t0, t0 + nt)
    const int t0 = (int)((int64_t)job.col16 * range / job.ranges);
    const int nt = (int)((int64_t)job.col16 * (range + 1) / job.ranges) - t0;
    const int nc = (H + kLmChunk - 1) / kLmChunk;                          // chunks per tile
    const int cpw = wave < nc ? (nc - 1 - wave) / kLmWaves + 1 : 0;        // this wave's
    const int nwv = nc < kLmWaves ? nc : kLmWaves;                         // waves with a chunk

    // (with one chunk per wave they stay for the whole pass; with more, each chunk reloads them)
    u32x4 afr[kLmSlices];
    if (cpw == 1) load_hidden_chunk(job, wave, lane, afr);

    // Loads of chunk wave + 8 j of tile t0 + ti: stg[r] = row r's 16 bytes at h = 512 c + 8 lane
    // (zero past H, and for rows past V: the descriptor ends at the last row, and reads past it
    // return zero without a memory access; for ti = nt the descriptor is empty, so a load may be
    // issued unconditionally, which keeps the compiler's waits for them exact).
    u32x4 stg[16];
    auto issue = [&](int ti, int j) {
        const int tv = 16 * (t0 + ti), c = wave + kLmWaves * j;
        const int rows = ti < nt ? min(16, V - tv) : 0;  // past the range: an empty descriptor
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(job.W + (int64_t)tv * H), (short)0, rows * H * 2, kBufWord3);
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

    // Epilogue of tile tt (waves 0..3): row 4 g + ei of its logits (the waves' partials added in
    // wave order), kept for a group of tiles and offered when the group is full or the range ends.
    auto epilogue = [&](int tt) {
        const float *pp = reinterpret_cast<const float *>(&part[tt & 1][0][lane]) + ei;
        float x = pp[0];
        for (int w = 1; w < nwv; ++w) x += pp[w * kWave * 4];
        const int slot = tt % kLmGroup;
#pragma unroll
        for (int c = 0; c < kLmGroup; ++c) xs[c] = slot == c ? x : xs[c];
        if (slot != kLmGroup - 1 && tt != nt - 1) return;
        // column (tb + c) * 16 + m for the group's tiles c <= slot
        const int tb = t0 + tt - slot;
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
    };

    // The chunk in stg to the wave's LDS area (the next loads may then reuse stg), and its 16
    // MFMAs over the fragments read back (same wave: LDS operations complete in order).
    auto stage_chunk = [&]() {
#pragma unroll
        for (int r = 0; r < 16; ++r) stage[wave][r][lane] = stg[r];
    };
    auto mma_chunk = [&](f32x4 &acc) {
#pragma unroll
        for (int s = 0; s < kLmSlices; ++s) {
            const u32x4 b = stage[wave][m][4 * s + g];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, afr[s]),
                                                          __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
        }
    };

    // Tile ti: its chunks' products while the next tile's loads are in flight, then (waves 0..3)
    // the previous tile's epilogue, still under those loads; the partial tile goes to buffer
    // ti % 2, which the epilogue of tile ti - 2 (before the last barrier) has finished reading.
    // Waves with one chunk (or none) and waves with several (H > 4096) run separate loops, so
    // that in the first no load writes the fragments and the MFMAs never wait for the loads in
    // flight.
    if (cpw <= 1) {
        for (int ti = 0; ti < nt; ++ti) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (cpw == 1) {
                stage_chunk();
                issue(ti + 1, 0);
                __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
                mma_chunk(acc);
            }
            if (ei < 4 && ti > 0) epilogue(ti - 1);
            if (cpw == 1) part[ti & 1][wave][lane] = acc;
            __syncthreads();
        }
    } else {
        for (int ti = 0; ti < nt; ++ti) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < cpw; ++j) {
                // (the next chunk's loads follow the MFMAs: the fragments and the loads in
                // flight are not live together, which keeps this path within the registers)
                stage_chunk();
                load_hidden_chunk(job, wave + kLmWaves * j, lane, afr);
                mma_chunk(acc);
                const bool more = j + 1 < cpw;
                issue(more ? ti : ti + 1, more ? j + 1 : 0);
            }
            if (ei < 4 && ti > 0) epilogue(ti - 1);
            part[ti & 1][wave][lane] = acc;
            __syncthreads();
        }
    }
    if (ei < 4 && nt > 0) epilogue(nt - 1);

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

// One wave per row merges the row's ranges (merge_row).
__global__ __launch_bounds__(kWave) void lmhead_merge_kernel(LmJob job) {
    __shared__ uint64_t pool[kLmPoolKeys + kWave / 2];  // keys >= T, then 64 range indices
    merge_row(job, (int)blockIdx.x, pool, (int)threadIdx.x);
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

// [R][ranges] lists, then [R][ranges] pairs.
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
    job.k = k;
    job.part_keys = static_cast<uint64_t *>(workspace);
    job.part_lse = reinterpret_cast<float2 *>(job.part_keys + (size_t)R * p.ranges * kLmList);
    job.cand_ids = cand_ids;
    job.unary = unary;
    job.lse_out = lse;
    if (R > 16) return hipErrorInvalidValue;  // the C ABI refuses these sizes
    hipLaunchKernelGGL(lmhead_topk_kernel, dim3((unsigned)job.ranges), dim3(kLmThreads), 0, stream,
                       job);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3((unsigned)R), dim3(kWave), 0, stream, job);
    return hipGetLastError();
}

}  // namespace dflash2
