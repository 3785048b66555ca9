// K1: per-row top-k + logsumexp over the full vocabulary (HBM-bound streaming pass).
//
// Computes, for every row of logits [R, V]: the first k tokens of the candidate order (higher
// logit first, equal logits by lower id) and unary_j = x_{cand_j} - logsumexp(row). Sources:
// "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector"
// (top 16 candidates per position; unary term U_t(b)); "DFlash2 Lands in llama.cpp" (ramgpt.org),
// section "What llama.cpp Actually Builds for the Selector" (per-position top-k, gathered unary).
//
// Design (gfx950, wave64):
//   * A row is cut into S slices (one workgroup each) and each slice into one contiguous range
//     per wave. Lanes read 16-byte vectors, consecutive lanes consecutive vectors (coalesced),
//     U vectors in flight per lane.
//   * logsumexp: each lane keeps an online (ref, sum) pair in the log2 domain; one v_exp per
//     element plus one rescale per batch.
//   * top-k: each wave keeps its 64 best keys sorted across its lanes (lane = rank). An element
//     is a candidate only if it beats the wave's current k-th key; the rare candidates are
//     compacted into a per-wave LDS staging list with ballot + popcount and merged into the
//     sorted list 64 at a time by a bitonic sort + merge across the lanes. The first full batch
//     seeds the threshold with the k-th largest of the 64 lane maxima (k real elements are at or
//     above it), so almost nothing is staged after the first batch.
//   * The waves' lists and (ref, sum) pairs are merged in fixed order: the result is
//     deterministic. With S > 1 a second kernel merges the slices in slice order.
#include "device_common.h"
#include "kernels.h"

namespace dflash2 {
namespace {

constexpr int kStageCap = 2 * kWave;  // staging list capacity per wave (keys)

struct WaveTopk {
    uint64_t top;      // this lane's entry of the wave's sorted list (lane = rank)
    uint64_t tau_key;  // admission threshold (wave-uniform): a key must exceed it
    float tau_v;       // logit of the threshold, for the cheap first test
    int cnt;           // staged keys (wave-uniform)
    uint64_t *stage;   // LDS [kStageCap]
    int k;
};

__device__ __forceinline__ void wave_flush(WaveTopk &w, int lane) {
    uint64_t c = lane < w.cnt ? w.stage[lane] : 0ull;
    c = wave_sort_desc(c, lane);
    w.top = wave_merge_desc(w.top, c, lane);
    const int rest = w.cnt - kWave;
    if (rest > 0) {
        const uint64_t t = lane < rest ? w.stage[kWave + lane] : 0ull;
        if (lane < rest) w.stage[lane] = t;
    }
    w.cnt = rest > 0 ? rest : 0;
    const uint64_t kth = __shfl(w.top, w.k - 1, kWave);
    if (kth != 0ull) {
        w.tau_key = kth;
        w.tau_v = key_logit(kth);
    }
}

// Stage `key` from every lane where `hit` holds; flush once 64 or more are staged.
__device__ __forceinline__ void wave_stage(WaveTopk &w, bool hit, uint64_t key, int lane) {
    const uint64_t mask = __ballot(hit);
    if (mask == 0ull) return;
    const int pos = w.cnt + __popcll(mask & ((1ull << lane) - 1ull));
    if (hit) w.stage[pos] = key;
    w.cnt += __popcll(mask);
    if (w.cnt >= kWave) wave_flush(w, lane);
}

// Offer NB elements per lane (ids id[j]) to the wave's top-k. `valid` masks padding lanes.
template <int NB>
__device__ __forceinline__ void offer(WaveTopk &w, const float *x, const int32_t *id,
                                      const bool *valid, float lane_max, int lane) {
    if (__ballot(lane_max >= w.tau_v) == 0ull) return;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const bool maybe = valid[j] && x[j] >= w.tau_v;
        if (__ballot(maybe) != 0ull) {
            const uint64_t key = cand_key(x[j], id[j]);
            wave_stage(w, maybe && key > w.tau_key, key, lane);
        }
    }
}

// One lane's online logsumexp update with NB elements, all valid.
template <int NB>
__device__ __forceinline__ void lse_update_full(float &ref, float &sum, const float *x, float bmax) {
    const float r = fmaxf(ref, bmax * kLog2e);
    sum *= __builtin_amdgcn_exp2f(ref - r);  // ref = -inf on the first batch: factor 0
    ref = r;
#pragma unroll
    for (int j = 0; j < NB; ++j) sum += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -r));
}

// Same with per-element validity (padding lanes and ragged ends).
template <int NB>
__device__ __forceinline__ void lse_update_masked(float &ref, float &sum, const float *x,
                                                  const bool *valid, float bmax) {
    if (bmax == -INFINITY) return;  // no valid element in this lane
    const float r = fmaxf(ref, bmax * kLog2e);
    if (ref != r) sum *= __builtin_amdgcn_exp2f(ref - r);
    ref = r;
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (valid[j]) sum += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -r));
}

template <typename T>
__device__ __forceinline__ u32x4 load_vec(const T *base, int64_t vec) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base) + vec);
}

template <typename T, int U>
__device__ __forceinline__ void load_batch(const T *logits, int64_t vbase, int lane, u32x4 *buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) buf[u] = load_vec(logits, vbase + lane + u * kWave);
}

// One full batch: U vectors per lane starting at vector vbase (+ lane + u * 64), all in the row.
template <typename T, int U, bool SEED>
__device__ __forceinline__ void full_batch(const u32x4 *buf, int64_t vbase, int64_t g0, int k,
                                           WaveTopk &w, float &ref, float &sum, int lane) {
    constexpr int EV = Elem<T>::kPerVec;
    constexpr int NB = U * EV;
    float x[NB];
#pragma unroll
    for (int u = 0; u < U; ++u) Elem<T>::unpack(buf[u], x + u * EV);
    float bmax = x[0];
#pragma unroll
    for (int j = 1; j < NB; ++j) bmax = fmaxf(bmax, x[j]);
    lse_update_full<NB>(ref, sum, x, bmax);
    if (SEED) {
        // Threshold seed: the k-th largest lane maximum (k real elements reach it).
        const uint64_t lk = wave_sort_desc((uint64_t)value_key(bmax) << 32, lane);
        w.tau_key = __shfl(lk, k - 1, kWave);
        w.tau_v = key_logit(w.tau_key);
    }
    int32_t id[NB];
    bool valid[NB];
    const int32_t id0 = (int32_t)((vbase + lane) * EV - g0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            id[u * EV + e] = id0 + u * kWave * EV + e;
            valid[u * EV + e] = true;
        }
    offer<NB>(w, x, id, valid, bmax, lane);
}

// Elements [e0, e1) of the flat tensor, one per lane per step (ragged row ends).
template <typename T>
__device__ __forceinline__ void scalar_range(const T *logits, int64_t e0, int64_t e1, int64_t row_start,
                             WaveTopk &w, float &ref, float &sum, int lane) {
    for (int64_t e = e0; e < e1; e += kWave) {
        const int64_t ei = e + lane;
        bool valid[1] = {ei < e1};
        float x[1] = {valid[0] ? Elem<T>::load(logits, ei) : -INFINITY};
        int32_t id[1] = {(int32_t)(ei - row_start)};
        lse_update_masked<1>(ref, sum, x, valid, x[0]);
        offer<1>(w, x, id, valid, x[0], lane);
    }
}

template <typename T, int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void topk_lse_kernel(
    const T *__restrict__ logits, int V, int k, int S, int32_t *__restrict__ cand_ids,
    float *__restrict__ unary, float *__restrict__ lse_out, uint64_t *__restrict__ part_keys,
    float2 *__restrict__ part_lse) {
    constexpr int EV = Elem<T>::kPerVec;
    constexpr int NB = U * EV;  // elements per lane per batch
    __shared__ uint64_t stage_all[WAVES][kStageCap];
    __shared__ uint64_t lists[WAVES][kWave];
    __shared__ float2 wave_lse[WAVES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t row = blockIdx.x / S;
    const int slice = blockIdx.x % S;

    // Full 16-byte vectors inside this row: [va, vb); ragged ends are handled element-wise.
    const int64_t g0 = row * (int64_t)V, g1 = g0 + V;
    int64_t va = (g0 + EV - 1) / EV, vb = g1 / EV;
    if (va > vb) va = vb = 0;
    const int64_t nvec = vb - va;
    const int chunks = S * WAVES, chunk = slice * WAVES + wave;
    const int64_t c0 = va + nvec * chunk / chunks, c1 = va + nvec * (chunk + 1) / chunks;

    WaveTopk w;
    w.top = 0ull;
    w.tau_key = 0ull;
    w.tau_v = -INFINITY;
    w.cnt = 0;
    w.stage = stage_all[wave];
    w.k = k;
    float ref = -INFINITY, sum = 0.0f;

    // Full batches (U vectors per lane), double-buffered: the next batch is in flight while the
    // current one is processed. The first batch also seeds the threshold.
    const int64_t step = (int64_t)U * kWave;
    const int64_t nfull = (c1 - c0) / step;
    int64_t vbase = c0 + nfull * step;
    if (nfull > 0) {
        u32x4 bufA[U], bufB[U];
        load_batch<T, U>(logits, c0, lane, bufA);
        if (nfull > 1) load_batch<T, U>(logits, c0 + step, lane, bufB);
        full_batch<T, U, true>(bufA, c0, g0, k, w, ref, sum, lane);
        for (int64_t b = 1; b < nfull; b += 2) {
            if (b + 1 < nfull) load_batch<T, U>(logits, c0 + (b + 1) * step, lane, bufA);
            full_batch<T, U, false>(bufB, c0 + b * step, g0, k, w, ref, sum, lane);
            if (b + 1 >= nfull) break;
            if (b + 2 < nfull) load_batch<T, U>(logits, c0 + (b + 2) * step, lane, bufB);
            full_batch<T, U, false>(bufA, c0 + (b + 1) * step, g0, k, w, ref, sum, lane);
        }
    }
    // Remaining vectors: one per lane per step.
    for (; vbase < c1; vbase += kWave) {
        const int64_t v = vbase + lane;
        const bool ok = v < c1;
        u32x4 raw = ok ? load_vec(logits, v) : u32x4{0u, 0u, 0u, 0u};
        float x[EV];
        Elem<T>::unpack(raw, x);
        int32_t id[EV];
        bool valid[EV];
        float bmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            valid[e] = ok;
            id[e] = (int32_t)(v * EV + e - g0);
            if (!ok) x[e] = -INFINITY;
            bmax = fmaxf(bmax, x[e]);
        }
        lse_update_masked<EV>(ref, sum, x, valid, bmax);
        offer<EV>(w, x, id, valid, bmax, lane);
    }
    // Ragged ends of the row (fewer than EV elements each, or the whole of a very short row).
    if (chunk == 0) scalar_range<T>(logits, g0, nvec > 0 ? va * EV : g1, g0, w, ref, sum, lane);
    if (chunk == chunks - 1 && nvec > 0) scalar_range<T>(logits, vb * EV, g1, g0, w, ref, sum, lane);
    if (w.cnt > 0) wave_flush(w, lane);

    // (ref, sum) across the wave, fixed butterfly order.
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const float oref = __shfl_xor(ref, off, kWave);
        const float osum = __shfl_xor(sum, off, kWave);
        lse_combine(ref, sum, oref, osum);
    }
    lists[wave][lane] = w.top;
    if (lane == 0) wave_lse[wave] = make_float2(ref, sum);
    __syncthreads();
    if (wave != 0) return;

    uint64_t acc = lists[0][lane];
    float2 ls = wave_lse[0];
    for (int q = 1; q < WAVES; ++q) {
        acc = wave_merge_desc(acc, lists[q][lane], lane);
        lse_combine(ls.x, ls.y, wave_lse[q].x, wave_lse[q].y);
    }
    if (S == 1) {
        const double lse = lse_value(ls.x, ls.y);
        if (lane < k) {
            cand_ids[row * k + lane] = key_id(acc);
            unary[row * k + lane] = (float)((double)key_logit(acc) - lse);
        }
        if (lane == 0 && lse_out) lse_out[row] = (float)lse;
    } else {
        part_keys[(row * S + slice) * kWave + lane] = acc;
        if (lane == 0) part_lse[row * S + slice] = ls;
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

template <typename T, int WAVES, int U>
hipError_t launch_k1(const TopkPlan &plan, const void *logits, int R, int V, int k,
                     int32_t *cand_ids, float *unary, float *lse, uint64_t *part_keys,
                     float2 *part_lse, hipStream_t stream) {
    const dim3 grid((unsigned)(R * plan.slices)), block(WAVES * kWave);
    hipLaunchKernelGGL((topk_lse_kernel<T, WAVES, U>), grid, block, 0, stream,
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
    TopkPlan p;
    p.waves = 4;
    // Enough workgroups to cover the chip, but at least ~4 full batches per wave.
    const int64_t target_wgs = 1024;
    const int64_t batch_elems = (int64_t)kWave * 4 * (16 / elem_bytes);
    const int64_t max_slices = (int64_t)V / (batch_elems * 4 * p.waves);
    int64_t s = (target_wgs + R - 1) / R;
    if (s > max_slices) s = max_slices;
    if (s < 1) s = 1;
    p.slices = (int)s;
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
        return launch_k1<float, 4, 4>(plan, logits, R, V, k, cand_ids, unary, lse, part_keys,
                                      part_lse, stream);
    return launch_k1<uint16_t, 4, 4>(plan, logits, R, V, k, cand_ids, unary, lse, part_keys,
                                     part_lse, stream);
}

}  // namespace dflash2
