// K1: per-row top-k + logsumexp over the full vocabulary (HBM-bound streaming pass).
//
// Computes, for every row of logits [R, V]: the first k tokens of the candidate order (higher
// logit first, equal logits by lower id) and unary_j = x_{cand_j} - logsumexp(row). Sources:
// "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector"
// (top 16 candidates per position; unary term U_t(b)); "DFlash2 Lands in llama.cpp" (ramgpt.org),
// section "What llama.cpp Actually Builds for the Selector" (per-position top-k, gathered unary).
//
// Design (gfx950, wave64): a workgroup of W waves per (row, slice); each wave streams its own
// contiguous part of the row. W is chosen so that about 16 waves share a CU (4 per SIMD): the
// SIMD then overlaps one wave's arithmetic with the other waves' loads. A row has S slices
// (S = 1 unless rows are too few to fill the chip; the slices are merged by a second kernel in
// slice order).
//   * Streaming: lanes read 16-byte vectors (consecutive lanes consecutive vectors) through a
//     buffer descriptor bounded to the wave's range, U vectors per lane per batch, NBUF - 1
//     batches issued ahead of the one processed.
//   * logsumexp: each lane keeps an online (ref, sum) pair in the log2 domain: one v_exp per
//     element plus one rescale per batch.
//   * top-k: each wave keeps its 64 best keys sorted across its lanes (lane = rank). An element
//     is admitted only if it beats the workgroup threshold: the largest k-th key any wave of the
//     workgroup holds, shared through LDS (each such key has k keys at or above it, so nothing
//     below it can be in the row's top k). A batch costs one compare per lane when no lane beats
//     it. Otherwise the lanes that do publish their raw batch to LDS and the wave reads each such
//     lane's elements back transposed (lane j <- element j). Each candidate is inserted straight
//     into the sorted list (rank by ballot + popcount, a one-lane DPP shift), and the wave's
//     k-th key is read back with readlane.
//   * The threshold starts at the k-th largest of the lane maxima of all the workgroup's waves
//     over their first NBUF - 1 batches (k real elements reach it).
//   * The waves' lists and (ref, sum) pairs are merged in wave order at the end.
// All orders are fixed and the merged top-k of distinct keys is unique, so results are
// deterministic.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kU = 4;     // 16-byte vectors per lane per batch
constexpr int kRing = 3;  // batches in flight per wave (kRing - 1 ahead of the one processed)
constexpr int kMaxWaves = 8;              // waves per workgroup (LDS: 4 KB each)
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family buffer descriptor word 3 (raw data)
constexpr int kNonTemporal = 2;           // cache policy: streaming data, read once
constexpr int kDppWaveShr1 = 0x138;       // DPP control: lane i reads lane i - 1

// Wave-uniform 64-bit broadcast of lane `src` (src uniform): two v_readlane, no LDS round trip.
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// Lane i receives lane i - 1's value (lane 0 receives 0).
__device__ __forceinline__ uint64_t shift_up_one(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, kDppWaveShr1, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), kDppWaveShr1, 0xF,
                                                    0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

struct WaveTopk {
    uint64_t top;      // this lane's entry of the wave's sorted list (lane = rank)
    uint64_t tau_key;  // admission threshold (wave-uniform): a key must exceed it
    float tau_v;       // logit of the threshold, for the cheap first test
    int k;
    uint64_t *shared_tau;  // the workgroup threshold in LDS
    uint64_t *pub;         // per wave of the workgroup: its list's n-th key (n = ceil(k / W))
    uint64_t pub_mine;     // what this wave last published
    int n, W, wave;
};

__device__ __forceinline__ void set_tau(WaveTopk &w, uint64_t key) {
    w.tau_key = key;
    w.tau_v = key_logit(key);
}

// The wave's own k-th key rose to `key`: adopt it and publish it to the workgroup.
__device__ __forceinline__ void raise_tau(WaveTopk &w, uint64_t key, int lane) {
    if (key > w.tau_key) {
        set_tau(w, key);
        if (lane == 0)
            __hip_atomic_fetch_max(w.shared_tau, key, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// Adopt the workgroup threshold if another wave has raised it past ours.
__device__ __forceinline__ void pull_tau(WaveTopk &w) {
    const uint64_t s = __hip_atomic_load(w.shared_tau, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
    // readfirstlane returns int: widen through uint32_t (no sign extension into the high half)
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)s);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(s >> 32));
    const uint64_t su = ((uint64_t)hi << 32) | lo;
    if (su > w.tau_key) set_tau(w, su);
}

// After a batch that changed the list: publish its n-th key and raise the workgroup threshold to
// the smallest n-th key over the W waves. Every wave has n distinct elements at or above its
// published key (a list position only ever grows), and W * n >= k, so k real elements reach
// that minimum: a valid threshold, usually well above the largest single-wave k-th key.
__device__ __forceinline__ void publish_and_refresh(WaveTopk &w, int lane) {
    const uint64_t mine = lane_value(w.top, w.n - 1);
    if (mine <= w.pub_mine) return;
    w.pub_mine = mine;
    if (lane == 0)
        __hip_atomic_store(&w.pub[w.wave], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // lane v reads wave v's key; the minimum is taken over wave-uniform values (scalar unit)
    const uint64_t p = lane < w.W ? __hip_atomic_load(&w.pub[lane], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_WORKGROUP)
                                  : ~0ull;
    uint64_t lo = mine;  // this wave's own value, not a stale read
    for (int v = 0; v < w.W; ++v) {
        if (v == w.wave) continue;
        const uint64_t o = lane_value(p, v);
        lo = o < lo ? o : lo;
    }
    raise_tau(w, lo, lane);
}

// Insert key c (wave-uniform, above the threshold) into the sorted list: its rank is the number
// of larger entries (a ballot), entries from that rank on move down one lane, and the threshold
// follows the wave's k-th key once k entries exist.
__device__ __forceinline__ void wave_insert(WaveTopk &w, uint64_t c, int lane) {
    const int p = __popcll(__ballot(w.top > c));
    const uint64_t prev = shift_up_one(w.top);
    w.top = lane < p ? w.top : (lane == p ? c : prev);
    raise_tau(w, lane_value(w.top, w.k - 1), lane);
}

// Offer a batch to the wave's top-k. Each lane holds U raw 16-byte vectors in `buf`, of which
// the first NSLOT elements are used; element j of lane L is real only if its vector
// (j / EV) * 64 + L is below `nvalid` (the raw words of the others may hold anything).
// `lane_max` is the largest real element of the lane. Element j of lane L has id
// id_base + L * lane_stride + (j / EV) * 64 * EV + (j % EV).
template <typename T, int U, int NSLOT>
__device__ __forceinline__ void offer_lanes(WaveTopk &w, const u32x4 *buf, float lane_max,
                                            bool lane_ok, int nvalid, int32_t id_base,
                                            int lane_stride, int lane, u32x4 *xbuf) {
    constexpr int EV = Elem<T>::kPerVec;
    static_assert(NSLOT <= kWave && NSLOT <= U * EV, "one element per lane in the transpose");
    const bool mine = lane_ok && lane_max >= w.tau_v;
    uint64_t hits = __ballot(mine);
    if (hits == 0ull) return;
    if (mine) {
#pragma unroll
        for (int u = 0; u < U; ++u) xbuf[lane * U + u] = buf[u];
    }
    const int j = lane;  // this lane reads element j of each publishing lane
    const int vec_j = (j / EV) * kWave;
    while (hits != 0ull) {
        const int L = __builtin_ctzll(hits);
        hits &= hits - 1ull;
        float x = -INFINITY;
        if (j < NSLOT) x = Elem<T>::lds_element(xbuf, L * U * EV + j);
        const bool maybe = j < NSLOT && vec_j + L < nvalid && x >= w.tau_v && x != -INFINITY;
        uint64_t m = __ballot(maybe);
        while (m != 0ull) {
            // each candidate's key is built from wave-uniform values (scalar unit)
            const int src = __builtin_ctzll(m);
            m &= m - 1ull;
            const float xs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), src));
            const int32_t id = id_base + L * lane_stride + (src / EV) * kWave * EV + (src % EV);
            const uint64_t c = cand_key(xs, id);
            if (c > w.tau_key) wave_insert(w, c, lane);
        }
    }
    publish_and_refresh(w, lane);
}

// One lane's online logsumexp update with NB elements (-inf elements add nothing).
template <int NB>
__device__ __forceinline__ void lse_update(float &ref, float &sum, const float *x, float bmax) {
    const float r = fmaxf(ref, bmax * kLog2e);
    sum *= __builtin_amdgcn_exp2f(ref - r);  // ref = -inf on the first batch: factor 0
    ref = r;
#pragma unroll
    for (int j = 0; j < NB; ++j) sum += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -r));
}

// One element, possibly absent (ragged ends and idle lanes).
__device__ __forceinline__ void lse_update_one(float &ref, float &sum, float x, bool valid) {
    if (!valid) return;
    const float r = fmaxf(ref, x * kLog2e);
    if (ref != r) sum *= __builtin_amdgcn_exp2f(ref - r);
    ref = r;
    sum += __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -r));
}

// U vectors of batch `b`: lane offset `voff` (fixed per lane) plus the wave-uniform batch offset;
// no per-lane address arithmetic. The descriptor bounds the wave's range: an offset past it
// reads zeros instead of memory.
template <int U>
__device__ __forceinline__ void load_batch(__amdgpu_buffer_rsrc_t rsrc, int voff, int b,
                                           u32x4 *buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        buf[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, (b * U + u) * kWave * 16,
                                                       kNonTemporal);
}

// Largest element per lane of a batch (only the first `nvalid` vectors are real).
template <typename T, int U, bool PARTIAL>
__device__ __forceinline__ void unpack_batch(const u32x4 *buf, int nvalid, int lane, float *x,
                                             float &bmax) {
    constexpr int EV = Elem<T>::kPerVec;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        Elem<T>::unpack(buf[u], x + u * EV);
        if (PARTIAL && u * kWave + lane >= nvalid) {
#pragma unroll
            for (int e = 0; e < EV; ++e) x[u * EV + e] = -INFINITY;
        }
    }
    bmax = x[0];
#pragma unroll
    for (int j = 1; j < U * EV; ++j) bmax = fmaxf(bmax, x[j]);
}

// One batch of the wave's range: vectors vbase + lane + u * 64. PARTIAL: only the first
// `nvalid` vectors are in range; the others (read as zeros) are replaced by -inf, which adds
// nothing to the sum and is never a candidate.
template <typename T, int U, bool PARTIAL>
__device__ __forceinline__ void batch(const u32x4 *buf, int64_t vbase, int64_t g0, int nvalid,
                                      WaveTopk &w, float &ref, float &sum, int lane,
                                      u32x4 *xbuf) {
    constexpr int EV = Elem<T>::kPerVec;
    constexpr int NB = U * EV;
    pull_tau(w);
    float x[NB], bmax;
    unpack_batch<T, U, PARTIAL>(buf, nvalid, lane, x, bmax);
    if (!PARTIAL || bmax != -INFINITY) lse_update<NB>(ref, sum, x, bmax);
    offer_lanes<T, U, (NB < kWave ? NB : kWave)>(w, buf, bmax, bmax != -INFINITY, nvalid,
                                                  (int32_t)(vbase * EV - g0), EV, lane, xbuf);
}

// Largest element of each lane over the batches already in the ring (the first NBUF - 1; the
// batch with index nfull is the partial one, with `tail` vectors). -inf for a lane with no data.
template <typename T, int U, int NBUF>
__device__ __forceinline__ float seed_lane_max(const u32x4 (*ring)[U], int nfull, int tail,
                                               int lane) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) {
        float x[U * Elem<T>::kPerVec], bmax = -INFINITY;
        if (i < nfull)
            unpack_batch<T, U, false>(ring[i], kWave * U, lane, x, bmax);
        else if (i == nfull && tail > 0)
            unpack_batch<T, U, true>(ring[i], tail, lane, x, bmax);
        m = fmaxf(m, bmax);
    }
    return m;
}

// The ragged ends of a row (its elements outside whole 16-byte vectors) hold fewer than 2 * EV
// elements: one per lane. They are loaded before the stream starts and offered after it.
template <typename T>
__device__ __forceinline__ float ragged_load(const T *logits, int64_t e0, int64_t e1, int lane) {
    const int64_t e = e0 + lane;
    return e < e1 ? Elem<T>::load(logits, e) : -INFINITY;
}

template <typename T>
__device__ __forceinline__ void ragged_offer(float x, int64_t e0, int64_t e1, int64_t g0,
                                             WaveTopk &w, float &ref, float &sum, int lane,
                                             u32x4 *xbuf) {
    const bool ok = e0 + lane < e1;
    lse_update_one(ref, sum, x, ok);
    const u32x4 raw = Elem<T>::single(x);
    offer_lanes<T, 1, 1>(w, &raw, x, ok, kWave, (int32_t)(e0 - g0), 1, lane, xbuf);
}

// Grid: R * S workgroups of W = blockDim.x / 64 waves; workgroup (row, slice) covers part
// slice of the row, wave w sub-part w of it.
template <typename T, int U, int NBUF>
__global__ __launch_bounds__(kWave * kMaxWaves) __attribute__((amdgpu_waves_per_eu(4))) void topk_lse_kernel(
    const T *__restrict__ logits, int V, int k, int S, int32_t *__restrict__ cand_ids,
    float *__restrict__ unary, float *__restrict__ lse_out, uint64_t *__restrict__ part_keys,
    float2 *__restrict__ part_lse) {
    constexpr int EV = Elem<T>::kPerVec;
    constexpr int step = U * kWave;  // vectors per batch
    extern __shared__ __attribute__((aligned(16))) u32x4 xbuf_all[];  // [W][64 * U]
    __shared__ uint64_t shared_tau;
    __shared__ float2 wave_lse[kMaxWaves];
    __shared__ uint32_t seed_vals[kMaxWaves * kWave];
    __shared__ uint64_t pub[kMaxWaves];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int W = blockDim.x / kWave;
    const int64_t row = blockIdx.x / S;
    const int slice = blockIdx.x % S;
    u32x4 *xbuf = xbuf_all + wave * (kWave * U);

    if (threadIdx.x == 0) shared_tau = 0ull;  // published to the other waves by the seed barrier
    if (threadIdx.x < kMaxWaves) pub[threadIdx.x] = 0ull;

    // Whole 16-byte vectors inside this row: [va, vb), split into S * W parts; this wave takes
    // part slice * W + wave: [c0, c1).
    const int64_t g0 = row * (int64_t)V, g1 = g0 + V;
    int64_t va = (g0 + EV - 1) / EV, vb = g1 / EV;
    if (va > vb) va = vb = 0;
    const int64_t nvec = vb - va;
    const int parts = S * W, part = slice * W + wave;
    const int64_t c0 = va + nvec * part / parts, c1 = va + nvec * (part + 1) / parts;
    const int64_t nv = c1 - c0;
    const int nfull = (int)(nv / step);
    const int tail = (int)(nv - (int64_t)nfull * step);  // vectors of the partial last batch

    WaveTopk w;
    w.top = 0ull;
    w.tau_key = 0ull;
    w.tau_v = -INFINITY;
    w.k = k;
    w.shared_tau = &shared_tau;
    w.pub = pub;
    w.pub_mine = 0ull;
    w.W = W;
    w.n = (k + W - 1) / W;
    w.wave = wave;
    float ref = -INFINITY, sum = 0.0f;

    // Ragged row ends (the first part takes the head, the last part the tail), loaded up front.
    const int64_t h0 = g0, h1 = nvec > 0 ? va * EV : g1, t0 = vb * EV, t1 = g1;
    const bool do_head = part == 0 && h1 > h0;
    const bool do_tail = part == parts - 1 && nvec > 0 && t1 > t0;
    const float xh = do_head ? ragged_load<T>(logits, h0, h1, lane) : -INFINITY;
    const float xt = do_tail ? ragged_load<T>(logits, t0, t1, lane) : -INFINITY;

    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(reinterpret_cast<const u32x4 *>(logits) + c0), 0, (int)(nv * 16),
        kBufferWord3);
    const int voff = lane * 16;

    // Batches (the last one partial when tail > 0) go through a ring of NBUF buffers, issued
    // NBUF - 1 batches ahead of the one processed; all NBUF are in flight during the seed.
    const int nall = nfull + (tail > 0 ? 1 : 0);
    u32x4 ring[NBUF][U];
#pragma unroll
    for (int i = 0; i < NBUF; ++i)
        if (i < nall) load_batch<U>(rsrc, voff, i, ring[i]);

    // Threshold seed: the k-th largest of the lane maxima of all waves over their first NBUF - 1
    // batches (k real elements reach it; -inf, which admits everything, when fewer than k lanes
    // hold data). The waves' ranges are disjoint, so the maxima are distinct elements. Found as
    // the largest order-preserving value key t with at least k maxima at or above it, one bit at
    // a time from the top with ballot counts: no cross-lane data movement.
    seed_vals[wave * kWave + lane] = value_key(seed_lane_max<T, U, NBUF>(ring, nfull, tail, lane));
    __syncthreads();
    {
        uint32_t v[kMaxWaves];
#pragma unroll
        for (int i = 0; i < kMaxWaves; ++i) v[i] = i < W ? seed_vals[i * kWave + lane] : 0u;
        uint32_t t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            int n = 0;
#pragma unroll
            for (int i = 0; i < kMaxWaves; ++i)
                if (i < W) n += __popcll(__ballot(v[i] >= c));
            if (n >= k) t = c;
        }
        raise_tau(w, (uint64_t)t << 32, lane);
    }

    for (int b0 = 0; b0 < nfull; b0 += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
            const int b = b0 + j;
            if (b >= nfull) break;
            if (b >= 1 && b + NBUF - 1 < nall)  // batch NBUF - 1 was loaded before the seed
                load_batch<U>(rsrc, voff, b + NBUF - 1, ring[(j + NBUF - 1) % NBUF]);
            batch<T, U, false>(ring[j], c0 + (int64_t)b * step, g0, step, w, ref, sum, lane, xbuf);
        }
    }
    if (tail > 0) {
        // the partial batch sits in ring slot nfull % NBUF (static register indexing)
#pragma unroll
        for (int j = 0; j < NBUF; ++j)
            if (j == nfull % NBUF)
                batch<T, U, true>(ring[j], c0 + (int64_t)nfull * step, g0, tail, w, ref, sum,
                                  lane, xbuf);
    }
    if (do_head) ragged_offer<T>(xh, h0, h1, g0, w, ref, sum, lane, xbuf);
    if (do_tail) ragged_offer<T>(xt, t0, t1, g0, w, ref, sum, lane, xbuf);

    // (ref, sum) across the wave, fixed butterfly order.
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const float oref = __shfl_xor(ref, off, kWave);
        const float osum = __shfl_xor(sum, off, kWave);
        lse_combine(ref, sum, oref, osum);
    }

    // Merge the waves' lists and pairs in wave order (wave 0 merges; lists staged in xbuf).
    uint64_t *lists = reinterpret_cast<uint64_t *>(xbuf_all);  // [W][64]
    __syncthreads();  // every wave is done with its xbuf
    lists[wave * kWave + lane] = w.top;
    if (lane == 0) wave_lse[wave] = make_float2(ref, sum);
    __syncthreads();
    if (wave != 0) return;
    uint64_t acc = w.top;
    for (int v = 1; v < W; ++v) {
        acc = wave_merge_desc(acc, lists[v * kWave + lane], lane);
        const float2 o = wave_lse[v];
        lse_combine(ref, sum, o.x, o.y);
    }
    if (S == 1) {
        const double lse = lse_value(ref, sum);
        if (lane < k) {
            cand_ids[row * k + lane] = key_id(acc);
            unary[row * k + lane] = (float)((double)key_logit(acc) - lse);
        }
        if (lane == 0 && lse_out) lse_out[row] = (float)lse;
    } else {
        part_keys[(row * S + slice) * kWave + lane] = acc;
        if (lane == 0) part_lse[row * S + slice] = make_float2(ref, sum);
    }
}

// Merge the S slice results of each row (one wave per row, slices in order).
__global__ __launch_bounds__(kWave) void topk_merge_kernel(
    int k, int S, const uint64_t *__restrict__ part_keys, const float2 *__restrict__ part_lse,
    int32_t *__restrict__ cand_ids, float *__restrict__ unary, float *__restrict__ lse_out) {
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    uint64_t acc = part_keys[row * S * kWave + lane];
    float2 ls = part_lse[row * S];
    for (int s = 1; s < S; ++s) {
        acc = wave_merge_desc(acc, part_keys[(row * S + s) * kWave + lane], lane);
        const float2 o = part_lse[row * S + s];
        lse_combine(ls.x, ls.y, o.x, o.y);
    }
    const double lse = lse_value(ls.x, ls.y);
    if (lane < k) {
        cand_ids[row * k + lane] = key_id(acc);
        unary[row * k + lane] = (float)((double)key_logit(acc) - lse);
    }
    if (lane == 0 && lse_out) lse_out[row] = (float)lse;
}

template <typename T>
hipError_t launch_k1(const TopkPlan &plan, const void *logits, int R, int V, int k,
                     int32_t *cand_ids, float *unary, float *lse, uint64_t *part_keys,
                     float2 *part_lse, hipStream_t stream) {
    const dim3 grid((unsigned)(R * plan.slices)), block(kWave * plan.waves);
    const size_t lds = (size_t)plan.waves * kWave * kU * sizeof(u32x4);
    hipLaunchKernelGGL((topk_lse_kernel<T, kU, kRing>), grid, block, lds, stream,
                       static_cast<const T *>(logits), V, k, plan.slices, cand_ids, unary, lse,
                       part_keys, part_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.slices == 1) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)R), dim3(kWave), 0, stream, k,
                       plan.slices, part_keys, part_lse, cand_ids, unary, lse);
    return hipGetLastError();
}

}  // namespace

TopkPlan plan_topk(int R, int V, int elem_bytes) {
    // About 4096 waves (16 per CU, 4 per SIMD), each streaming at least 2 batches: as many waves
    // per row as that allows (up to kMaxWaves in one workgroup), then slices if rows are still too few.
    const int64_t target_waves = 4096;
    const int64_t batch_elems = (int64_t)kWave * kU * (16 / elem_bytes);
    int64_t max_parts = (int64_t)V / (batch_elems * 2);
    if (max_parts < 1) max_parts = 1;
    int64_t want = (target_waves + R - 1) / R;
    if (want > max_parts) want = max_parts;
    if (want < 1) want = 1;
    TopkPlan p;
    p.waves = 1;
    while (p.waves * 2 <= want && p.waves * 2 <= kMaxWaves) p.waves *= 2;
    p.slices = (int)((want + p.waves - 1) / p.waves);
    if ((int64_t)p.slices * p.waves > max_parts) p.slices = (int)(max_parts / p.waves);
    if (p.slices < 1) p.slices = 1;
    return p;
}

size_t topk_workspace_bytes(const TopkPlan &p, int R) {
    if (p.slices <= 1) return 0;
    return (size_t)R * p.slices * (kWave * sizeof(uint64_t) + sizeof(float2));
}

hipError_t launch_topk_lse(const void *logits, int logits_dtype, int R, int V, int k,
                           int32_t *cand_ids, float *unary, float *lse, void *workspace,
                           hipStream_t stream) {
    const TopkPlan plan = plan_topk(R, V, logits_dtype == 0 ? 4 : 2);
    uint64_t *part_keys = static_cast<uint64_t *>(workspace);
    float2 *part_lse = reinterpret_cast<float2 *>(part_keys + (size_t)R * plan.slices * kWave);
    if (logits_dtype == 0)
        return launch_k1<float>(plan, logits, R, V, k, cand_ids, unary, lse, part_keys, part_lse,
                                stream);
    return launch_k1<uint16_t>(plan, logits, R, V, k, cand_ids, unary, lse, part_keys, part_lse,
                               stream);
}

}  // namespace dflash2
