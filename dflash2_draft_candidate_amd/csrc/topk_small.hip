// K1 for few rows: per-row top-k + logsumexp when the rows are too few to fill the chip (decode
// at batch 1 and other small batches), with the slices of a row merged inside the same kernel.
//
// Computes what topk_lse.hip computes (sources there): per row of logits [R, V], the first k
// tokens of the candidate order (higher logit first, equal logits by lower id, +0 == -0), their
// unary scores x - logsumexp(row) and the row's logsumexp.
//
// Design (gfx950, wave64). Each row is cut into S slices, and all slices of all rows are
// resident at once (at most one 1024-thread workgroup per CU). A workgroup reads its slice in one
// round trip (every thread issues all of its 16-byte vector loads before it uses any). This pass
// is latency-bound: a lone wave on a SIMD waits about ten cycles between dependent VALU
// instructions, so the sixteen waves (four per SIMD) hide each other's latency, and each step
// keeps the instructions per element few.
//   * logsumexp: each thread sums exp2(x log2e - ref) against its own largest element (the
//     reference), which is exact for any finite input; the (ref, sum) pairs are combined by a
//     fixed lane tree, then a fixed tree over the waves, then over the slices: deterministic.
//   * top-k: the slice's threshold is the k-th largest of a set of lane maxima (k real elements
//     reach it): of each wave's 64 (a sort of them) and of the sixteen waves' four largest. Its
//     elements at or above it (one float compare each) are compacted into LDS, and sorted by
//     waves 64 at a time, then merged. With very many (ties, flat slices) each wave's lanes offer
//     them in rounds, largest first, one sort and merge per round, and the wave lists are merged.
//   * slices: each slice writes its list and pair to the workspace with device-scope atomic
//     stores (coherent across the XCDs' L2 caches), waits for them to complete and then counts
//     itself in the row's arrival counter; the slice whose count completes the row reads the
//     partials back with device-scope atomic loads, merges them (a tree over its waves) and writes
//     the outputs. Device-scope release / acquire fences are not used: on gfx950 they write back
//     or invalidate the whole L2 of the XCD, which cost more than the pass itself. The counter
//     holds a launch epoch above the count: epochs grow from launch to launch, so an atomic max
//     at the start re-bases a counter left by an earlier launch, and the last slice clears the
//     count, so replays of a captured launch (same epoch) start from zero. Nothing waits on
//     another workgroup.
//   * gate (optional): workgroups past the slices compute split-K tiles of hidden . W_sel with
//     the stand-alone gate kernel's decomposition and summation order (gate_tile.h; its first
//     four waves), so a fused selector call reproduces the stage-by-stage gate bit for bit.
#include "arrival.h"
#include "device_common.h"
#include "gate_tile.h"
#include "kernels.h"
#include "row_slices.h"

namespace dflash2 {
namespace {

constexpr int kSmWaves = 16;
constexpr int kSmThreads = kSmWaves * kWave;
constexpr int kSmVec = 4;            // 16-byte vectors per thread at most (one load round)
constexpr int kSmMaxSlices = 64;     // slices per row at most (the merge reads S lists)
constexpr int kSmTargetWgs = 256;    // workgroups resident at once (one per CU)
constexpr int kSmSliceWgs = 128;     // slice workgroups the plan aims at: at 16 rows of 151936,
                                     // 8 slices a row (12.0 us) beat 5, 6, 10, 12 and 16 (12.1-12.7)
constexpr int kSmMinVecs = 64;       // a slice keeps at least this many vectors
constexpr int kSmMaxNt = 8;          // gate tiles of up to 8 x 16 columns ride along
constexpr int kSmCand = 4 * kWave;   // candidates a slice compacts for sorting, at most
constexpr int kBufWord3 = 0x00020000;  // gfx9-family buffer descriptor word 3 (raw data)
constexpr int kNonTemp = 2;            // cache policy: streaming data, read once

struct SmallGate {
    const uint16_t *hidden;  // [R, H] bf16
    const uint16_t *W;       // [H, r] bf16
    float *part;             // [splits][R][r]
    int R, H, r, mtiles, splits;
};

struct SmallShared {
    uint64_t lists[kSmWaves][kWave];  // sorted lists: candidate chunks, wave lists, merge tree
    uint64_t cand[kSmCand + kWave];   // compacted (logit bits, id) pairs, then a discard slot per lane
    float2 pairs[kSmWaves];
    uint32_t tw[kSmWaves];            // each wave's threshold (value key)
    uint32_t top4[kSmWaves * 4];      // each wave's four largest lane maxima (value keys)
    uint32_t ncand_all;
    uint32_t last;                    // this workgroup's slice arrived last
};

// Out-of-line sort and merge (several waves call them; one copy of the code).
__device__ __attribute__((noinline)) uint64_t sort_keys(uint64_t key, int lane) {
    return wave_sort_desc(key, lane);
}
__device__ __attribute__((noinline)) uint64_t merge_keys(uint64_t a, uint64_t c, int lane) {
    return wave_merge_desc(a, c, lane);
}

__device__ __forceinline__ uint64_t pick64(uint64_t v, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of 32-bit lane values into descending lane order.
template <int S>
__device__ __forceinline__ uint32_t u32_merge_steps(uint32_t v, int lane, bool desc) {
    const uint32_t o = xor_lane<S>(v, lane);
    const bool keep_max = ((lane & S) == 0) == desc;
    v = ((v > o) == keep_max) ? v : o;
    if constexpr (S > 1) v = u32_merge_steps<S / 2>(v, lane, desc);
    return v;
}
__device__ __forceinline__ uint32_t u32_sort_desc(uint32_t v, int lane) {
    v = u32_merge_steps<1>(v, lane, (lane & 2) == 0);
    v = u32_merge_steps<2>(v, lane, (lane & 4) == 0);
    v = u32_merge_steps<4>(v, lane, (lane & 8) == 0);
    v = u32_merge_steps<8>(v, lane, (lane & 16) == 0);
    v = u32_merge_steps<16>(v, lane, (lane & 32) == 0);
    return u32_merge_steps<32>(v, lane, true);
}

// (ref, sum) combination as lse_combine, with the hardware exp2 (the scale factors lie in (0, 1]).
__device__ __forceinline__ void pair_combine(float &ref, float &sum, float oref, float osum) {
    const float r = fmaxf(ref, oref);
    const float a = ref == r ? sum : sum * __builtin_amdgcn_exp2f(ref - r);
    const float b = oref == r ? osum : osum * __builtin_amdgcn_exp2f(oref - r);
    ref = r;
    sum = a + b;
}

template <int S>
__device__ __forceinline__ void pair_step(float &ref, float &sum, int lane) {
    const float orf = __uint_as_float(xor_lane<S>(__float_as_uint(ref), lane));
    const float osm = __uint_as_float(xor_lane<S>(__float_as_uint(sum), lane));
    pair_combine(ref, sum, orf, osm);
}

// (ref, sum) of every lane combined by a fixed xor tree: every lane ends with the same pair.
__device__ __forceinline__ void wave_pair(float &ref, float &sum, int lane) {
    pair_step<1>(ref, sum, lane);
    pair_step<2>(ref, sum, lane);
    pair_step<4>(ref, sum, lane);
    pair_step<8>(ref, sum, lane);
    pair_step<16>(ref, sum, lane);
    pair_step<32>(ref, sum, lane);
}

// This thread's elements: vector i (i < kSmVec) if it lies in the slice, then the ragged head and
// tail element (wave 0 only; -inf where absent). for_each skips a vector that no lane of the wave
// holds.
template <typename T>
struct ThreadElems {
    static constexpr int EV = Elem<T>::kPerVec;
    u32x4 raw[kSmVec];
    float xh, xt;
    int nmine;           // vectors of this thread (the first nmine of raw)
    int32_t id_vec0;     // id of element 0 of vector 0 (vector i adds i * kSmThreads * EV)
    int32_t id_h, id_t;  // ids of the head / tail element

    template <typename F>
    __device__ __forceinline__ void for_each(bool ragged, F &&f) const {
#pragma unroll
        for (int i = 0; i < kSmVec; ++i)
            if (i < nmine) {
                float x[EV];
                Elem<T>::unpack(raw[i], x);
#pragma unroll
                for (int e = 0; e < EV; ++e) f(x[e], id_vec0 + i * kSmThreads * EV + e);
            }
        if (ragged) {
            f(xh, id_h);
            f(xt, id_t);
        }
    }
};

// The candidate key of the compacted (logit bits, id) pair in a written slot (the pair of logit
// +0 at id 0 is all zero bits, so zero cannot mark an empty slot).
__device__ __forceinline__ uint64_t pair_key(uint64_t p) {
    return cand_key(__uint_as_float((uint32_t)(p >> 32)), (int32_t)(uint32_t)p);
}

// One gate tile (tile t = split sp * mtiles + m-tile mt): the first four waves compute it with the
// stand-alone gate kernel's ranges and summation order; every wave takes part in the barrier and
// the store.
template <int NT>
__device__ void gate_tile(const SmallGate &gj, int t, int wave, int lane, float *red) {
    constexpr int PITCH = gate_pitch<NT>();
    constexpr int GW = gate_waves<NT>();
    const int mt = t % gj.mtiles, sp = t / gj.mtiles;
    if (wave < GW) {
        int s0, s1;
        gate_steps(gj.H, sp * GW + wave, gj.splits * GW, s0, s1);
        f32x4 acc[NT];
        gate_wave<NT>(gj.hidden, gj.W, gj.R, gj.H, gj.r, mt * 16, s0, s1, lane, acc);
        const int m = lane & 15, g = lane >> 4;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[(wave * 16 + g * 4 + i) * PITCH + out_col<NT>(tt, m)] = acc[tt][i];
    }
    __syncthreads();
    float *dst = gj.part + (int64_t)sp * gj.R * gj.r;
    for (int e = threadIdx.x; e < 16 * gj.r; e += kSmThreads) {
        const int rr = e / gj.r, c = e % gj.r, orow = mt * 16 + rr;
        if (orow >= gj.R) continue;
        float v = red[rr * PITCH + c];
#pragma unroll
        for (int w = 1; w < GW; ++w) v += red[(w * 16 + rr) * PITCH + c];
        dst[(int64_t)orow * gj.r + c] = v;
    }
}

template <int NT>
constexpr size_t gate_red_floats_small() {
    return NT == 0 ? 1 : (size_t)gate_waves<NT>() * 16 * gate_pitch<NT>();
}

// Waves [h, 2h) hand their lists to waves [0, h), which merge them, for h = top, top / 2, ..., 1:
// wave 0 ends with the merge of the first 2 * top waves' lists.
__device__ __forceinline__ uint64_t tree_merge(SmallShared &sh, uint64_t list, int top, int wave,
                                               int lane) {
#pragma unroll 1
    for (int h = top; h >= 1; h >>= 1) {
        if (wave >= h && wave < 2 * h) sh.lists[wave][lane] = list;
        __syncthreads();
        if (wave < h) list = merge_keys(list, sh.lists[wave + h][lane], lane);
    }
    return list;
}

// Grid: R * S slice workgroups, then (NTG > 0) gj.mtiles * gj.splits gate workgroups.
template <typename T, int NTG>
__global__ __launch_bounds__(kSmThreads) void topk_small_kernel(
    const T *__restrict__ logits, int V, int k, int S, int n_units, uint32_t epoch,
    int32_t *__restrict__ cand_ids, float *__restrict__ unary, float *__restrict__ lse_out,
    uint64_t *__restrict__ part_keys, float2 *__restrict__ part_lse,
    uint64_t *__restrict__ arrivals, SmallGate gj) {
    constexpr int EV = Elem<T>::kPerVec;
    __shared__ SmallShared sh;
    __shared__ float red[gate_red_floats_small<NTG>()];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    if ((int)blockIdx.x >= n_units) {
        if constexpr (NTG > 0) gate_tile<NTG>(gj, (int)blockIdx.x - n_units, wave, lane, red);
        return;
    }

    // ---- one load round: every vector of this thread's share of the slice ----
    const int unit = blockIdx.x;
    const UnitRange ur = unit_range(unit, V, S, EV);
    ThreadElems<T> te;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(reinterpret_cast<const u32x4 *>(logits) + ur.c0), 0, ur.nv * 16,
        kBufWord3);
    te.nmine = 0;
#pragma unroll
    for (int i = 0; i < kSmVec; ++i) {
        // (vectors past the slice read as zero and are not used; the wave skips a load that no
        // lane needs)
        if (i * kSmThreads < ur.nv)
            te.raw[i] = __builtin_amdgcn_raw_buffer_load_b128(
                rsrc, ((int)threadIdx.x + i * kSmThreads) * 16, 0, kNonTemp);
        te.nmine += (int)threadIdx.x + i * kSmThreads < ur.nv ? 1 : 0;
    }
    // Launch epochs grow, so an atomic max of (epoch, 0) re-bases a counter left by an earlier
    // launch and leaves one of this launch alone; it is not waited for.
    const int64_t row = unit / S;
    if (S > 1 && threadIdx.x == 0) arrival_rebase(&arrivals[row], epoch);
    te.xh = te.xt = -INFINITY;
    const bool ragged = wave == 0 && (ur.h1 > ur.h0 || ur.t1 > ur.t0);
    if (ragged) {  // the ragged ends hold fewer than 2 * EV elements
        if (ur.h0 + lane < ur.h1) te.xh = Elem<T>::load(logits, ur.h0 + lane);
        if (ur.t0 + lane < ur.t1) te.xt = Elem<T>::load(logits, ur.t0 + lane);
    }
    te.id_vec0 = (int32_t)((ur.c0 + threadIdx.x) * EV - ur.g0);
    te.id_h = (int32_t)(ur.h0 - ur.g0) + lane;
    te.id_t = (int32_t)(ur.t0 - ur.g0) + lane;

    // ---- this thread's largest element and its (ref, sum) pair ----
    float mx = -INFINITY;
    te.for_each(ragged, [&](float x, int32_t) { mx = fmaxf(mx, x); });
    float ref = mx == -INFINITY ? -INFINITY : mx * kLog2e;
    float sum = 0.f;
    if (mx != -INFINITY)
        te.for_each(ragged, [&](float x, int32_t) {
            sum += __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -ref));
        });
    wave_pair(ref, sum, lane);

    // ---- the slice's candidates ----
    // The threshold is the k-th largest of a set of lane maxima (k real elements reach it): each
    // wave's own 64, and the 64 made of every wave's four largest (the tighter one when few
    // threads share the slice's top elements); the largest of these holds for the slice.
    // (the readlane stays outside lane-dependent branches: inside one, the compiler may replace
    // its operand by what that operand equals in the branch's own lanes)
    const uint32_t smk = u32_sort_desc(mx == -INFINITY ? 0u : value_key(mx), lane);
    const uint32_t tw = __builtin_amdgcn_readlane(smk, k - 1);
    if (lane < 4) sh.top4[wave * 4 + lane] = smk;
    if (lane == 0) {
        sh.tw[wave] = tw;
        sh.pairs[wave] = make_float2(ref, sum);
    }
    if (threadIdx.x == 0) sh.ncand_all = 0u;
    __syncthreads();
    uint32_t tv = __builtin_amdgcn_readlane(u32_sort_desc(sh.top4[lane], lane), k - 1);
#pragma unroll
    for (int w = 0; w < kSmWaves; ++w) tv = max(tv, sh.tw[w]);
    // Value keys and logits order alike (+0 == -0), so the test is one float compare; with no
    // threshold (fewer than k lanes hold an element) every element but -inf passes.
    const float tf = tv == 0u ? -3.40282347e+38f : key_value(tv);  // -FLT_MAX
    // (a wave none of whose lane maxima reaches the threshold holds no candidate)
    if (__ballot(mx >= tf) != 0ull) {
        uint32_t cnt = 0u;
        te.for_each(ragged, [&](float x, int32_t) { cnt += x >= tf ? 1u : 0u; });
        // compacted into one buffer as (logit bits, id) pairs (the order is irrelevant: a sort
        // follows), without branches: a lane's other elements, and all of them once the buffer
        // is full, go to its discard slot
        uint32_t pos = 0u;
        if (cnt) pos = atomicAdd(&sh.ncand_all, cnt);
        const bool fits = pos + cnt <= (uint32_t)kSmCand;
        te.for_each(ragged, [&](float x, int32_t id) {
            const bool c = fits && x >= tf;
            sh.cand[c ? pos : (uint32_t)(kSmCand + lane)] =
                ((uint64_t)__float_as_uint(x) << 32) | (uint32_t)id;
            pos += c ? 1u : 0u;
        });
    }
    __syncthreads();
    const uint32_t total = sh.ncand_all;
    uint64_t list = 0ull;
    if (total <= (uint32_t)kSmCand) {
        // the usual case: wave c sorts candidates 64c .. 64c + 63, and wave 0 merges the chunks
        const int nch = (int)(total + kWave - 1) / kWave;
        if (wave < nch) {
            const int i = wave * kWave + lane;
            list = sort_keys(i < (int)total ? pair_key(sh.cand[i]) : 0ull, lane);
        }
        if (nch > 1) {
            if (wave < nch) sh.lists[wave][lane] = list;
            __syncthreads();
            if (wave == 0) {
#pragma unroll 1
                for (int c = 1; c < nch; ++c) list = merge_keys(list, sh.lists[c][lane], lane);
            }
        }
    } else {
        // many candidates (ties, flat slices): in rounds, every lane offers its largest candidate
        // below the one it offered last and above its wave list's k-th key; one sort and merge
        // per round (every round takes a key from each lane still offering, so this ends); the
        // wave lists are merged
        uint64_t lt = 0ull;
        uint64_t cap = ~0ull;
        for (;;) {
            uint64_t best = 0ull;
            te.for_each(ragged, [&](float x, int32_t id) {
                const uint64_t key = x >= tf ? cand_key(x, id) : 0ull;
                if (key < cap && key > lt && key > best) best = key;
            });
            if (__ballot(best != 0ull) == 0ull) break;
            list = merge_keys(list, sort_keys(best, lane), lane);
            lt = pick64(list, k - 1);
            cap = best;
        }
        list = tree_merge(sh, list, kSmWaves / 2, wave, lane);
    }

    // ---- the slice's list and pair (pairs in a fixed tree over the waves) ----
    if (wave == 0) {
        // Publish the list first (a device-scope atomic store: coherent across the XCDs' L2
        // caches), so that its write overlaps the pair tree.
        if (S > 1)
            __hip_atomic_store(&part_keys[(int64_t)unit * kWave + lane], list, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        float r0 = -INFINITY, s0 = 0.f;
        if (lane < kSmWaves) {
            r0 = sh.pairs[lane].x;
            s0 = sh.pairs[lane].y;
        }
        static_assert(kSmWaves == 16, "the pair tree spans 16 lanes");
        pair_step<1>(r0, s0, lane);
        pair_step<2>(r0, s0, lane);
        pair_step<4>(r0, s0, lane);
        pair_step<8>(r0, s0, lane);  // lanes 0 .. 15 hold the slice's pair: lane 0's to all
        r0 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(r0)));
        s0 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s0)));
        if (S == 1) {
            const double lse = lse_value(r0, s0);
            if (lane < k) {
                cand_ids[row * k + lane] = key_id(list);
                unary[row * k + lane] = (float)((double)key_logit(list) - lse);
            }
            if (lane == 0 && lse_out) lse_out[row] = (float)lse;
        } else {
            // Publish the pair as the list; count the arrival only once both stores have
            // completed, which orders them before the count without a release fence (that writes
            // back the whole L2).
            if (lane == 0)
                __hip_atomic_store(reinterpret_cast<uint64_t *>(&part_lse[unit]),
                                   ((uint64_t)__float_as_uint(s0) << 32) | __float_as_uint(r0),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            stores_complete();
            if (lane == 0) sh.last = arrive(&arrivals[row], epoch, (uint32_t)S) ? 1u : 0u;
        }
    }
    if (S == 1) return;
    __syncthreads();
    if (sh.last == 0u) return;

    // ---- the last slice: merge the row's S lists and pairs, write the outputs ----
    // Every slice's partial was complete before it counted itself; the loads are device-scope
    // atomic loads, which bypass stale lines in this XCD's L2. Lane i of wave w loads entry i < k
    // of the lists of slices w, w + 16, ... (entries past k cannot reach the row's first k) and
    // merges them; then the waves' lists are merged in a tree.
    constexpr int kPer = kSmMaxSlices / kSmWaves;
    const uint64_t *pk = part_keys + row * S * kWave;
    uint64_t got[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int sl = wave + i * kSmWaves;
        got[i] = sl < S && lane < k ? __hip_atomic_load(&pk[sl * kWave + lane], __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0ull;
    }
    uint64_t pp = 0ull;
    if (wave == 0 && lane < S)
        pp = __hip_atomic_load(reinterpret_cast<uint64_t *>(&part_lse[row * S + lane]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    list = got[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i)
        if (wave + i * kSmWaves < S) list = merge_keys(list, got[i], lane);
    int top = 1;  // the waves holding lists: min(S, 16), merged in a tree
    while (2 * top < min(S, kSmWaves)) top *= 2;
    list = tree_merge(sh, list, top, wave, lane);
    if (wave != 0) return;
    float pr = -INFINITY, ps = 0.f;
    if (lane < S) {
        pr = __uint_as_float((uint32_t)pp);
        ps = __uint_as_float((uint32_t)(pp >> 32));
    }
    wave_pair(pr, ps, lane);
    const double lse = lse_value(pr, ps);
    if (lane < k) {
        cand_ids[row * k + lane] = key_id(list);
        unary[row * k + lane] = (float)((double)key_logit(list) - lse);
    }
    if (lane == 0) {
        if (lse_out) lse_out[row] = (float)lse;
        // every slice of this launch has counted itself: clear the count for a replay of the
        // same launch (same epoch)
        arrival_clear(&arrivals[row], epoch);
    }
}

template <typename T, int NTG>
void launch_small_t(const SmallPlanInfo &p, const void *logits, int R, int V, int k,
                    uint32_t epoch, int32_t *cand_ids, float *unary, float *lse, void *workspace,
                    const SmallGate &gj, hipStream_t stream) {
    const int units = R * p.slices;
    uint64_t *keys = static_cast<uint64_t *>(workspace);
    float2 *pairs = reinterpret_cast<float2 *>(keys + (size_t)units * kWave);
    uint64_t *arr = reinterpret_cast<uint64_t *>(pairs + units);
    const int grid = units + (NTG > 0 ? gj.mtiles * gj.splits : 0);
    hipLaunchKernelGGL((topk_small_kernel<T, NTG>), dim3((unsigned)grid), dim3(kSmThreads), 0,
                       stream, static_cast<const T *>(logits), V, k, p.slices, units, epoch,
                       cand_ids, unary, lse, keys, pairs, arr, gj);
}

template <typename T>
void launch_small_g(const SmallPlanInfo &p, int nt, const void *logits, int R, int V, int k,
                    uint32_t epoch, int32_t *cand_ids, float *unary, float *lse, void *workspace,
                    const SmallGate &gj, hipStream_t stream) {
    switch (nt) {
    case 1: launch_small_t<T, 1>(p, logits, R, V, k, epoch, cand_ids, unary, lse, workspace, gj, stream); break;
    case 2: launch_small_t<T, 2>(p, logits, R, V, k, epoch, cand_ids, unary, lse, workspace, gj, stream); break;
    case 4: launch_small_t<T, 4>(p, logits, R, V, k, epoch, cand_ids, unary, lse, workspace, gj, stream); break;
    case 8: launch_small_t<T, 8>(p, logits, R, V, k, epoch, cand_ids, unary, lse, workspace, gj, stream); break;
    default: launch_small_t<T, 0>(p, logits, R, V, k, epoch, cand_ids, unary, lse, workspace, gj, stream); break;
    }
}

}  // namespace

bool plan_small(int R, int V, int elem_bytes, SmallPlanInfo &p) {
    if (R < 1 || R >= kSmTargetWgs) return false;
    const int64_t EV = 16 / elem_bytes;
    const int64_t nvec = V / EV + 1;      // whole vectors of a row, at most
    const int64_t per_wg = (int64_t)kSmThreads * kSmVec;
    const int64_t s_need = (nvec + per_wg - 1) / per_wg;
    // every slice resident at once (one workgroup per CU), one load round each; otherwise the
    // streaming pass
    if (s_need > kSmMaxSlices || R * s_need > kSmTargetWgs) return false;
    // a row that one workgroup covers with a vector per thread stays whole: splitting it would
    // save less than the slice merge costs (a store, an arrival and a load round trip)
    if (nvec <= kSmThreads) {
        p.slices = 1;
        return true;
    }
    int64_t s = kSmSliceWgs / R;
    const int64_t s_cap = nvec / kSmMinVecs;
    if (s > s_cap) s = s_cap;
    if (s > kSmMaxSlices) s = kSmMaxSlices;
    if (s < s_need) s = s_need;
    p.slices = (int)(s < 1 ? 1 : s);
    return true;
}

size_t small_workspace_bytes(const SmallPlanInfo &p, int R) {
    if (p.slices <= 1) return 0;
    const size_t units = (size_t)R * p.slices;
    return units * kWave * sizeof(uint64_t) + units * sizeof(float2) + (size_t)R * sizeof(uint64_t);
}

int small_gate_nt(int r) {
    const int nt = (r + 15) / 16;
    if (nt > kSmMaxNt) return 0;
    return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8;
}

hipError_t launch_topk_small(const SmallPlanInfo &p, const void *logits, int logits_dtype, int R,
                             int V, int k, uint32_t epoch, int32_t *cand_ids, float *unary,
                             float *lse, void *workspace, hipStream_t stream,
                             const FusedGate *gate) {
    SmallGate gj{};
    int nt = 0;
    if (gate) {
        nt = small_gate_nt(gate->r);
        if (nt == 0) return hipErrorInvalidValue;
        gj.hidden = static_cast<const uint16_t *>(gate->hidden);
        gj.W = static_cast<const uint16_t *>(gate->W_sel);
        gj.part = gate->part;
        gj.R = R;
        gj.H = gate->H;
        gj.r = gate->r;
        gj.mtiles = (R + 15) / 16;
        gj.splits = gate_splits(R, gate->H, 1);
    }
    if (logits_dtype == 0)
        launch_small_g<float>(p, nt, logits, R, V, k, epoch, cand_ids, unary, lse, workspace, gj,
                              stream);
    else
        launch_small_g<uint16_t>(p, nt, logits, R, V, k, epoch, cand_ids, unary, lse, workspace,
                                 gj, stream);
    return hipGetLastError();
}

}  // namespace dflash2
