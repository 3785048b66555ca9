// K1: per-row top-k + logsumexp over the full vocabulary (HBM-bound streaming pass).
//
// Computes, for every row of logits [R, V]: the first k tokens of the candidate order (higher
// logit first, equal logits by lower id) and unary_j = x_{cand_j} - logsumexp(row). Sources:
// "DFlash 2: Keep Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector"
// (top 16 candidates per position; unary term U_t(b)); "DFlash2 Lands in llama.cpp" (ramgpt.org),
// section "What llama.cpp Actually Builds for the Selector" (per-position top-k, gathered unary).
//
// Design (gfx950, wave64). A unit is a (row, slice) pair (S slices per row; S = 1 unless rows
// are too few to fill the chip, and then a second kernel merges the slices in slice order). Two
// workgroups of 8 waves share a CU (each owns G <= 4 units; W = 8 / G waves stream each unit):
// a workgroup whose units are done leaves its SIMDs to the other one, which one 16-wave
// workgroup per CU could not do (its waves waited for its slowest unit).
//   * Balance. The SIMD issues oldest-first, so with a static split the youngest wave on each
//     SIMD finished far behind the oldest. Here a unit's waves share the unit's chunks (CB
//     batches of 4 vectors per lane) through an LDS counter, so a favoured wave simply takes
//     more chunks, and a wave whose unit has none left helps another unit of its workgroup.
//   * Streaming. Lanes read 16-byte vectors (consecutive lanes, consecutive vectors) through a
//     buffer descriptor bounded to the unit (an offset past it reads zeros), with a ring of
//     kRing batches in registers, kRing - 1 issued ahead of the one processed.
//   * logsumexp with a fixed reference. Each lane sums 2^(x log2e) (a reference of 0 in the log2
//     domain: one v_exp per element, no per-batch rescale) over a chunk and stores the sum to
//     LDS; the sums are added per lane in chunk order at the end, so the result does not depend
//     on which wave took which chunk. A chunk whose sum leaves the safe fp32 range (logits above
//     about 69) or a row total too small to keep its precision sends the unit down a slow exact
//     path at the end.
//   * top-k. A 64-bit key (order-preserving logit map above the inverted id) makes the candidate
//     order one unsigned compare. The unit's oldest wave (its owner) keeps the unit's 64 best
//     keys sorted across its lanes; the other waves queue their candidates to it through LDS,
//     each element set in consecutive slots reserved with one atomic add (a wave waits for
//     room if the owner is a lap behind; the owner always catches up). An element is admitted
//     only if it beats the unit's threshold in LDS, which is always valid (k real elements at
//     or above it): the k-th key of the owner's list, or the seed below. A batch costs one
//     compare per lane of the lane's term sum unless it reaches the threshold's term; then the
//     batch's flagged vectors (by their own sums, or their maxima in near-flat rows) are staged
//     in LDS together and read back transposed (lane i <- staged element i), and the owner
//     inserts each surviving candidate by ballot + popcount rank and a one-lane DPP shift.
//     After its stream the owner takes what is queued 64 at a time and, when more than a few
//     pass the threshold, sorts them and merges the two sorted lists.
//   * Seed. The threshold starts at the k-th largest of the lane maxima of the unit's waves over
//     their first batches (k real elements reach it); with more than four waves per unit, the
//     k-th largest of the lane-wise maxima over the waves (one search instead of one per
//     wave, so small units get it before most of their batches are read).
//   * End. The owner keeps draining the queue until every wave of its unit has finished the
//     stream; after a barrier each wave adds a fixed range of the unit's chunk sums, and the
//     owner takes what is left in the queue, adds the partial sums in wave order and writes the
//     results (the top k of distinct keys is unique, whatever the order they arrived in).
//     Deterministic throughout.
//   * Fused gate (bf16 activations, r <= 128). The selector's gate product is independent of
//     the logits, so the top-k pass can carry it: workgroup t computes split-K tile t of
//     hidden . W_sel (the same tiles, wave ranges and summation order as the stand-alone gate
//     kernel) on four of its waves (one per SIMD) before they join the stream; the last of the
//     four to finish sums their parts through LDS and stores the tile. The work sharing lets the
//     other twelve waves absorb the delay. A gate rides along only where its tile parts fit in
//     LDS beside the chunk sums of the pass's own plan (so select and the stage-by-stage calls
//     sum the same chunks). Tiles are numbered XCD by XCD (see gate_tile_of).
#include <atomic>

#include "device_common.h"
#include "gate_tile.h"
#include "kernels.h"
#include "row_slices.h"

namespace dflash2 {
namespace {

constexpr int kU = 4;                     // 16-byte vectors per lane per batch
constexpr int kStep = kU * kWave;         // vectors per batch
constexpr int kRing = 3;                  // batch buffers per wave (kRing - 1 loads ahead)
constexpr int kWaves = 8;                 // waves per workgroup: two workgroups fill a CU
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxUnits = 4;              // units per workgroup (W = kWaves / G >= 2)
constexpr int kTargetWorkgroups = 512;    // two per CU
constexpr int kSliceBelowRows = 256;      // fewer rows than this are cut into slices
constexpr int kMinBatchesPerWave = 1;     // slices are not cut smaller than this per wave
constexpr size_t kLdsBudget = 56 * 1024;  // chunk sums per workgroup (dynamic LDS)
constexpr size_t kLdsDynamicMax = 66 * 1024;  // chunk sums + a fused gate's tile parts
constexpr float kSumLimit = 0x1p100f;     // a chunk sum above this leaves the fast path
constexpr float kSumFloor = 0x1p-60f;     // so does a unit total below this
constexpr float kTermMargin = 1.f - 0x1p-10f;  // v_exp_f32 is far more accurate than this
constexpr int kMaxSumHits = 8;            // lanes the sum filter may flag before maxima decide
constexpr int kQueueSlots = 512;          // candidate queue slots per workgroup (G units share)
constexpr int kSeedBatches = 3;           // batches per wave behind the seed (<= kRing)
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family buffer descriptor word 3 (raw data)
constexpr int kNonTemporal = 2;           // cache policy: streaming data, read once
constexpr int kDppWaveShr1 = 0x138;       // DPP control: lane i reads lane i - 1

// Wave-uniform 64-bit broadcast of lane `src` (src uniform): two v_readlane, no LDS round trip.
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// A value every lane holds (read back from LDS) as a wave-uniform value. readfirstlane returns
// int: widen through uint32_t (no sign extension into the high half).
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Lane i receives lane i - 1's value (lane 0 receives 0: it has no source, and the bound
// control writes zero there, with no cleared destination needed).
__device__ __forceinline__ uint64_t shift_up_one(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, kDppWaveShr1, 0xF, 0xF,
                                                           true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kDppWaveShr1,
                                                           0xF, 0xF, true);
    return ((uint64_t)hi << 32) | lo;
}

// Per-workgroup state in LDS (besides the chunk sums).
struct K1Shared {
    uint64_t tau[kMaxUnits];          // admission threshold of each unit
    uint64_t queue[kQueueSlots];      // candidates on their way to the units' owners (0: empty);
                                      // unit q owns slots [q, q + 1) * kQueueSlots / G
    uint32_t q_tail[kMaxUnits];       // queue slots reserved so far
    uint32_t q_head[kMaxUnits];       // queue slots consumed by the owner so far
    alignas(16) float vstage[kWaves][128];  // each wave's flagged vectors staged by a batch
    uint32_t seed_vals[kWaves * kWave];  // seed maxima; after the stream: partial chunk sums
    float rag[kMaxUnits * kWave];     // the unit's ragged-end sums per lane
    u32x4 stage[kWaves][kU];          // per wave: one hit lane's batch, read back transposed
    uint32_t next_chunk[kMaxUnits];   // next chunk of the unit to hand out
    uint32_t seeded[kMaxUnits];       // waves of the unit that have published their seed
    uint32_t seed_done[kMaxUnits];    // the unit's seed is in tau
    uint32_t overflow[kMaxUnits];     // a chunk sum left the safe range
    uint32_t gate_arrived;            // gate waves that have stored their part of the tile
    int64_t unit_c0[kMaxUnits];       // each unit's first whole vector,
    int32_t unit_nv[kMaxUnits];       // its whole vectors,
    int32_t unit_idb0[kMaxUnits];     // the id of its first vector's first element,
    uint32_t unit_nch[kMaxUnits];     // and its chunks (0: no unit)
    uint32_t done_all;                // waves that have finished the stream
};
static_assert(sizeof(K1Shared) + kLdsDynamicMax <= 80 * 1024,
              "two workgroups share the 160 KB of LDS of a CU (gfx950)");

static_assert(kLdsDynamicMax >= kLdsBudget, "the chunk sums always fit");

// The gate tiles carried by the top-k pass: tile t = sp * mtiles + mt covers rows mt*16 ..
// mt*16 + 15 over split sp of H, written to part[sp][R][r].
struct GateJob {
    const uint16_t *hidden;  // [R, H] bf16
    const uint16_t *W;       // [H, r] bf16
    float *part;             // [splits][R][r]
    int R, H, r, mtiles, splits;
};

// The gate waves: slots 4-7, one per SIMD, none of them a unit's owner (owners are the slots
// below G <= 4).
template <int G> constexpr int gate_first_wave() { return 4; }

template <int NT>
constexpr size_t gate_red_floats() {
    return NT == 0 ? 0 : (size_t)gate_waves<NT>() * 16 * gate_pitch<NT>();
}

// Workgroups are dispatched to the XCDs round-robin (workgroup g on XCD g % kXcds). Numbering
// the gate tiles XCD by XCD gives each XCD a run of consecutive tiles (m-tiles of one or two
// W_sel slices), so each XCD's L2 fetches the W_sel slices it needs once instead of every
// XCD fetching all of W_sel for every m-tile.
constexpr int kXcds = 8;
// The gate tile of workgroup g of n (-1: none) when there are T <= n tiles: the first
// T / kXcds workgroups of each XCD take that XCD's run of consecutive tiles, so the tiles spread
// evenly over the XCDs (and, dispatched first, over the CUs).
__device__ __forceinline__ int gate_tile_of(int g, int n, int T) {
    if (T % kXcds != 0 || n % kXcds != 0) return g < T ? g : -1;
    const int j = g / kXcds;
    return j < T / kXcds ? (g % kXcds) * (T / kXcds) + j : -1;
}

// Wave gw (0..3) of the workgroup's gate tile; the last of the four stores the tile.
template <int NT>
__device__ __forceinline__ void gate_tile_part(const GateJob &gj, int gw, int lane, float *red,
                                            uint32_t *arrived) {
    constexpr int PITCH = gate_pitch<NT>();
    const int t = gate_tile_of(blockIdx.x, gridDim.x, gj.mtiles * gj.splits);
    if (t < 0) return;
    const int mt = t % gj.mtiles, sp = t / gj.mtiles;
    int s0, s1;
    constexpr int GW = gate_waves<NT>();
    gate_steps(gj.H, sp * GW + gw, gj.splits * GW, s0, s1);
    f32x4 acc[NT];
    // (four steps of loads in flight up to 4 column tiles: the stream's registers are not live
    // yet; at 8 tiles two would spill)
    gate_wave<NT, NT <= 4 ? 4 : batch_steps<NT>(), NT <= 4>(gj.hidden, gj.W, gj.R, gj.H, gj.r,
                                                              mt * 16, s0, s1, lane, acc);
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(gw * 16 + g * 4 + i) * PITCH + out_col<NT>(tt, m)] = acc[tt][i];
    uint32_t a = 0u;
    if (lane == 0)
        a = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(a) != GW - 1) return;
    // the last of the four: every part is in LDS; add them in wave order
    float *dst = gj.part + (int64_t)sp * gj.R * gj.r;
    for (int e = lane; e < 16 * gj.r; e += kWave) {
        const int rr = e / gj.r, c = e % gj.r, orow = mt * 16 + rr;
        if (orow >= gj.R) continue;
        float v = red[rr * PITCH + c];
#pragma unroll
        for (int w = 1; w < GW; ++w) v += red[(w * 16 + rr) * PITCH + c];
        dst[(int64_t)orow * gj.r + c] = v;
    }
}

struct WaveTopk {
    uint64_t top;          // this lane's entry of the wave's sorted list (lane = rank): the
                           // unit's list for its owner, an overflow list for the others
    uint64_t tau_key;      // admission threshold (wave-uniform): a key must exceed it
    float tau_v;           // logit of the threshold, for the cheap first test
    int k;
    uint64_t *shared_tau;  // the unit's threshold in LDS
    uint64_t *queue;       // the unit's candidate queue (qmask + 1 slots, a power of two)
    uint32_t *q_tail, *q_head;
    uint32_t qmask;
    uint32_t head;         // owner: slots consumed
    bool owner;            // this wave keeps the unit's list
    bool home;             // the unit being processed is the wave's own (else it helps another)
};

// Key 0 (no threshold yet) admits every element: its logit is -inf, not the NaN the key map
// would give (a NaN threshold would fail every comparison and drop candidates).
__device__ __forceinline__ void set_tau(WaveTopk &w, uint64_t key) {
    w.tau_key = key;
    w.tau_v = key == 0ull ? -INFINITY : key_logit(key);
}

// A valid threshold `key` was found: adopt it and publish it to the unit.
__device__ __forceinline__ void raise_tau(WaveTopk &w, uint64_t key, int lane) {
    if (key > w.tau_key) {
        set_tau(w, key);
        if (lane == 0)
            __hip_atomic_fetch_max(w.shared_tau, key, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// The unit's current threshold (other waves may have raised it).
__device__ __forceinline__ void pull_tau(WaveTopk &w) {
    const uint64_t s = uniform64(__hip_atomic_load(w.shared_tau, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP));
    if (s > w.tau_key) set_tau(w, s);
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

// Candidates above which a set is sorted and merged into the list in one go instead of being
// inserted one at a time (a bitonic sort and merge cost about as much as this many inserts).
constexpr int kBulkInsert = 6;

// Add the candidates c (one per lane, 0 = none; every nonzero one above the threshold) to the
// wave's list: one insert at a time, or (BULK, for many) sort them and merge the two sorted
// lists (the 64 largest keys of both; keys are distinct, so the result is the same either
// way). The sort holds too many registers for the stream loop, so only the owner's drain after
// the stream uses it.
template <bool BULK>
__device__ __forceinline__ void insert_set(WaveTopk &w, uint64_t c, int lane) {
    uint64_t m = __ballot(c != 0ull);
    if (BULK && __popcll(m) > kBulkInsert) {
        w.top = wave_merge_desc(w.top, wave_sort_desc(c, lane), lane);
        raise_tau(w, lane_value(w.top, w.k - 1), lane);
        return;
    }
    while (m != 0ull) {
        const int src = __builtin_ctzll(m);
        m &= m - 1ull;
        const uint64_t cs = lane_value(c, src);
        if (cs > w.tau_key) wave_insert(w, cs, lane);
    }
}

// Reserve n consecutive queue slots (one atomic add) and wait until the owner has consumed what
// they held a lap before. The owner takes the queue in order and keeps doing so until every wave
// of the workgroup is done, so the wait ends; a reserved slot is always written afterwards (the
// owner stops at a slot not yet written).
__device__ __forceinline__ uint32_t reserve_slots(WaveTopk &w, int lane, uint32_t n) {
    uint32_t p = 0u;
    if (lane == 0) {
        p = __hip_atomic_fetch_add(w.q_tail, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        uint32_t head =
            __hip_atomic_load(w.q_head, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (p + n - head > w.qmask + 1u) {
            __builtin_amdgcn_s_sleep(1);
            head = __hip_atomic_load(w.q_head, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    return __builtin_amdgcn_readfirstlane(p);
}

// Candidates of one element position set: the lanes in m hold one each, with key `key`. The
// owner inserts them into its list one by one; another wave queues them to the owner in
// consecutive slots reserved at once.
__device__ __forceinline__ void emit_keys(WaveTopk &w, uint64_t m, uint64_t key, int lane) {
    if (!w.owner) {
        const uint32_t pos = reserve_slots(w, lane, (uint32_t)__popcll(m));
        if ((m >> lane) & 1ull) {
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            __hip_atomic_store(&w.queue[(pos + rank) & w.qmask], key, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        return;
    }
    while (m != 0ull) {
        const int src = __builtin_ctzll(m);
        m &= m - 1ull;
        const uint64_t c = lane_value(key, src);
        if (c > w.tau_key) wave_insert(w, c, lane);
    }
}

// Owner: insert the queued candidates, consuming the written prefix of the queue (a reserved
// slot not yet written stops it until the next call). `all`: after the stream, when every
// reserved slot is written: take them all. BULK: sort and merge large sets (see insert_set).
template <bool BULK>
__device__ __forceinline__ void drain(WaveTopk &w, int lane, bool all) {
    const uint32_t tail = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(w.q_tail, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
    while (w.head != tail) {
        const uint32_t n = min(tail - w.head, (uint32_t)kWave);
        const uint32_t slot = (w.head + lane) & w.qmask;
        const uint64_t key = lane < (int)n ? __hip_atomic_load(&w.queue[slot], __ATOMIC_ACQUIRE,
                                                               __HIP_MEMORY_SCOPE_WORKGROUP)
                                           : 0ull;
        const uint64_t written = __ballot(key != 0ull);
        uint32_t cnt = n;
        if (!all) {  // the prefix of written slots
            const uint64_t gaps = ~written & (n >= 64 ? ~0ull : ((1ull << n) - 1ull));
            cnt = gaps ? (uint32_t)__builtin_ctzll(gaps) : n;
        }
        if (cnt == 0u) return;
        insert_set<BULK>(w, lane < (int)cnt && key > w.tau_key ? key : 0ull, lane);
        if (lane < (int)cnt)
            __hip_atomic_store(&w.queue[slot], 0ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        w.head += cnt;
        if (lane == 0)
            __hip_atomic_store(w.q_head, w.head, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (cnt < n) return;
    }
}

// Offer a batch to the wave's list. Each lane holds U raw 16-byte vectors in `buf`, of which
// the first NSLOT elements are used; element j of lane L is real only if its vector
// (j / EV) * 64 + L is below `nvalid` (the raw words of the others may hold anything). `hits`
// holds every lane that may have an element at or above the threshold (a superset is fine:
// each element is compared exactly). Element j of lane L has id
// id_base + L * lane_stride + (j / EV) * 64 * EV + (j % EV).
template <typename T, int U, int NSLOT>
__device__ __forceinline__ void offer_lanes(WaveTopk &w, const u32x4 *buf, uint64_t hits,
                                            int nvalid, int32_t id_base, int lane_stride,
                                            int lane, u32x4 *stage) {
    constexpr int EV = Elem<T>::kPerVec;
    static_assert(NSLOT <= kWave && NSLOT <= U * EV, "one element per lane in the transpose");
    if (hits == 0ull) return;
    const int j = lane;  // this lane reads element j of each hit lane
    const int vec_j = (j / EV) * kWave;
    while (hits != 0ull) {
        const int L = __builtin_ctzll(hits);
        hits &= hits - 1ull;
        if (lane == L) {
#pragma unroll
            for (int u = 0; u < U; ++u) stage[u] = buf[u];
        }
        float x = -INFINITY;
        if (j < NSLOT) x = Elem<T>::lds_element(stage, j);
        const bool maybe = j < NSLOT && vec_j + L < nvalid && x >= w.tau_v && x != -INFINITY;
        const uint64_t m = __ballot(maybe);
        if (m != 0ull)
            emit_keys(w, m, cand_key(x, id_base + L * lane_stride + (j / EV) * kWave * EV + (j % EV)),
                      lane);
    }
}

// Batch `b` of a unit: lane offset `voff` (fixed per lane) plus the wave-uniform batch offset.
// The descriptor bounds the unit: an offset past it reads zeros instead of memory.
__device__ __forceinline__ void load_batch(__amdgpu_buffer_rsrc_t rsrc, int voff, int b,
                                           u32x4 *buf) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
        buf[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, (b * kU + u) * kWave * 16,
                                                       kNonTemporal);
}

// Elements of a batch and the largest per lane (only the first `nvalid` vectors are real; the
// others become -inf, which adds nothing to a sum and is never a candidate).
template <typename T, bool PARTIAL>
__device__ __forceinline__ void unpack_batch(const u32x4 *buf, int nvalid, int lane, float *x,
                                             float &bmax) {
    constexpr int EV = Elem<T>::kPerVec;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        Elem<T>::unpack(buf[u], x + u * EV);
        if (PARTIAL && u * kWave + lane >= nvalid) {
#pragma unroll
            for (int e = 0; e < EV; ++e) x[u * EV + e] = -INFINITY;
        }
    }
    bmax = x[0];
#pragma unroll
    for (int j = 1; j < kU * EV; ++j) bmax = fmaxf(bmax, x[j]);
}

// Vectors staged at once by a batch's candidate pass (as floats: kStageVecs * kVecElems of them
// per wave, in its row of K1Shared::vstage).
constexpr int kStageVecs = 16;
constexpr int kVecElems = 8;  // floats per staged vector (a 16-byte vector of bf16)
static_assert(kStageVecs * kVecElems == 128, "K1Shared::vstage holds one stage per wave");
static_assert(kStageVecs * 4 <= kU * 16, "the staged vectors' ids fit the wave's stage");

// One batch: add its terms 2^(x log2e - R) to the lane's chunk sum and offer it to the list.
// Each lane sums its kU vectors separately and adds the four sums in a fixed order. A vector's
// sum is at least its largest term, so a vector whose sum is below the threshold's term
// (t_e = 2^(tau log2e - R), less a margin for exp2's rounding) holds no candidate, and no
// maximum is needed. When t_e underflows to 0, or the sums flag more than kMaxSumHits lanes
// (near-flat rows, where every sum is large), each vector's maximum decides instead. The
// flagged vectors (as floats) are staged in the wave's LDS area kStageVecs at a time, in rank
// order, and read back transposed (lane i <- staged element i), so one staging round trip
// serves the whole batch; each element at or above the threshold is handed on (emit_keys).
template <typename T, bool PARTIAL>
__device__ __forceinline__ void batch(const u32x4 *buf, int nvalid, int32_t id_base, float R,
                                      float t_e, float &csum, WaveTopk &w, int lane,
                                      float *vstage, int32_t *vid) {
    constexpr int EV = Elem<T>::kPerVec;
    constexpr int NB = kU * EV;
    static_assert(kU == 4, "the vector sums are added as (s0 + s1) + (s2 + s3)");
    static_assert(EV <= kVecElems, "a staged vector holds a 16-byte vector's elements");
    float x[NB];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        Elem<T>::unpack(buf[u], x + u * EV);
        if (PARTIAL && u * kWave + lane >= nvalid) {
#pragma unroll
            for (int e = 0; e < EV; ++e) x[u * EV + e] = -INFINITY;
        }
    }
    float vs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        vs[u] = __builtin_amdgcn_exp2f(fmaf(x[u * EV], kLog2e, -R));
#pragma unroll
        for (int e = 1; e < EV; ++e) vs[u] += __builtin_amdgcn_exp2f(fmaf(x[u * EV + e], kLog2e, -R));
    }
    const float bs = (vs[0] + vs[1]) + (vs[2] + vs[3]);
    csum += bs;
    // (the lane sum is at least each vector sum, so the lanes test first)
    const uint64_t any = __ballot(bs >= t_e);
    if (any == 0ull && t_e != 0.f) return;
    // bit u: vector u may hold a candidate
    uint32_t fl = (vs[0] >= t_e ? 1u : 0u) | (vs[1] >= t_e ? 2u : 0u) |
                  (vs[2] >= t_e ? 4u : 0u) | (vs[3] >= t_e ? 8u : 0u);
    if (t_e == 0.f || __popcll(any) > kMaxSumHits) {
        // the sums do not single out a few lanes (e.g. near-flat rows): the vectors' maxima
        fl = 0u;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float vm = x[u * EV];
#pragma unroll
            for (int e = 1; e < EV; ++e) vm = fmaxf(vm, x[u * EV + e]);
            fl |= (vm != -INFINITY && vm >= w.tau_v) ? (1u << u) : 0u;
        }
    }
    uint32_t P = 0u;  // flagged vectors
#pragma unroll
    for (int u = 0; u < kU; ++u) P += (uint32_t)__popcll(__ballot((fl >> u) & 1u));
    for (uint32_t r0 = 0u; r0 < P; r0 += kStageVecs) {
        // rank of a flagged vector: those of lower u first, then by lane; ranks r0 ... go now
        uint32_t below = 0u;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint64_t hu = __ballot((fl >> u) & 1u);
            const uint32_t r = below - r0 + __builtin_amdgcn_mbcnt_hi(
                                                (uint32_t)(hu >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)hu, 0u));
            if (((fl >> u) & 1u) && r < (uint32_t)kStageVecs) {  // (r wraps below r0)
#pragma unroll
                for (int e = 0; e < EV; e += 4)
                    *reinterpret_cast<f32x4 *>(vstage + r * kVecElems + e) =
                        f32x4{x[u * EV + e], x[u * EV + e + 1], x[u * EV + e + 2],
                              x[u * EV + e + 3]};
                vid[r] = id_base + (u * kWave + lane) * EV;
            }
            below += (uint32_t)__popcll(hu);
        }
        const uint32_t nv_st = min(P - r0, (uint32_t)kStageVecs);
        for (uint32_t base = 0u; base < nv_st * kVecElems; base += kWave) {
            const uint32_t i = base + (uint32_t)lane;
            const uint32_t v = i / kVecElems, e = i % kVecElems;
            float xi = -INFINITY;
            int32_t id = 0;
            if (v < nv_st && e < (uint32_t)EV) {
                xi = vstage[i];
                id = vid[v] + (int32_t)e;
            }
            const uint64_t m = __ballot(xi >= w.tau_v && xi != -INFINITY);
            if (m != 0ull) emit_keys(w, m, cand_key(xi, id), lane);
        }
    }
}

// Unit q and index wv within the unit of wave slot s, mixing the SIMD age classes (slot s sits
// on SIMD s % 4 with age s / 4) so that every unit gets the same mix; and the inverse.
template <int G>
__device__ __forceinline__ void wave_unit(int s, int &q, int &wv) {
    q = s % G;
    wv = s / G;
}
template <int G>
__device__ __forceinline__ int unit_slot(int q, int wv) {
    return q + G * wv;
}

// The exact logsumexp pair of a unit's elements with a per-lane online reference (slow path,
// one wave, used only when a chunk sum left the fast path's range).
template <typename T>
__device__ void exact_pair(const T *logits, const UnitRange &u, int lane, float &ref,
                           float &sum) {
    constexpr int EV = Elem<T>::kPerVec;
    ref = -INFINITY;
    sum = 0.f;
    auto add = [&](float x) {
        const float r = fmaxf(ref, x * kLog2e);
        sum = sum * __builtin_amdgcn_exp2f(ref - r) + __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -r));
        ref = r;
    };
    for (int64_t e = u.h0 + lane; e < u.h1; e += kWave) add(Elem<T>::load(logits, e));
    for (int64_t e = u.c0 * EV + lane; e < (u.c0 + u.nv) * EV; e += kWave)
        add(Elem<T>::load(logits, e));
    for (int64_t e = u.t0 + lane; e < u.t1; e += kWave) add(Elem<T>::load(logits, e));
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const float oref = __shfl_xor(ref, off, kWave);
        const float osum = __shfl_xor(sum, off, kWave);
        lse_combine(ref, sum, oref, osum);
    }
}

// Grid: ceil(units / G) workgroups of kWaves waves; workgroup g owns units g*G .. g*G + G - 1
// (and gate tile g, if NTG > 0 and g < mtiles * splits). Dynamic LDS: the chunk sums
// [G][nch_max][64] floats, then the gate's per-wave tiles [4][16][NTG * 16 + 1] floats.
template <typename T, int G, int NTG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
topk_lse_kernel(const T *__restrict__ logits, int V, int k, int S, int n_units, int CB,
                int nch_max, int32_t *__restrict__ cand_ids, float *__restrict__ unary,
                float *__restrict__ lse_out, uint64_t *__restrict__ part_keys,
                float2 *__restrict__ part_lse, GateJob gj) {
    constexpr int EV = Elem<T>::kPerVec;
    extern __shared__ __attribute__((aligned(16))) float chunk_sums[];
    __shared__ K1Shared sh;

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int W = kWaves / G;
    int q, wv;
    wave_unit<G>(wave, q, wv);
    const int64_t unit = (int64_t)blockIdx.x * G + q;
    const bool active = unit < n_units;  // trailing units of the last workgroup idle
    const UnitRange ur = unit_range(active ? unit : 0, V, S, EV);
    const int nv = active ? ur.nv : 0;
    const int nb = (nv + kStep - 1) / kStep;  // batches of the unit
    const int nch = (nb + CB - 1) / CB;       // chunks of the unit
    const int P = (kRing + CB - 1) / CB;      // chunks per wave assigned up front
    float *csums = chunk_sums + (size_t)q * nch_max * kWave;
    u32x4 *stage = sh.stage[wave];
    // flagged vectors staged by a batch (floats) and their first ids (in the wave's stage,
    // which the ragged ends use only before the stream)
    float *vstage = sh.vstage[wave];
    int32_t *vid = reinterpret_cast<int32_t *>(sh.stage[wave]);

    if (threadIdx.x < kMaxUnits) {
        sh.tau[threadIdx.x] = 0ull;
        sh.next_chunk[threadIdx.x] = (uint32_t)(W * P);
        sh.overflow[threadIdx.x] = 0u;
    }
    if (threadIdx.x < kMaxUnits) sh.q_tail[threadIdx.x] = sh.q_head[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < kQueueSlots; i += kThreads) sh.queue[i] = 0ull;
    if (threadIdx.x < kMaxUnits) sh.seeded[threadIdx.x] = sh.seed_done[threadIdx.x] = 0u;
    if (threadIdx.x == 0) sh.gate_arrived = sh.done_all = 0u;
    if (wv == 0 && lane == 0) {
        sh.unit_c0[q] = ur.c0;
        sh.unit_nv[q] = nv;
        sh.unit_idb0[q] = (int32_t)(ur.c0 * EV - ur.g0);
        sh.unit_nch[q] = (uint32_t)nch;
    }
    __syncthreads();  // the only barrier before the stream (every wave arrives long before data)

    if constexpr (NTG > 0) {
        if (wave >= gate_first_wave<G>() && wave < gate_first_wave<G>() + gate_waves<NTG>())
            gate_tile_part<NTG>(gj, wave - gate_first_wave<G>(), lane,
                                chunk_sums + (size_t)G * nch_max * kWave, &sh.gate_arrived);
    }

    const int voff = lane * 16;
    // Issue side: the unit being loaded (the wave's own; once it has no chunks left, a wave other
    // than the owner helps the unit of the workgroup with the most chunks left).
    int iq = q, i_nb = nb, i_nch = nch;
    __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(reinterpret_cast<const u32x4 *>(logits) + ur.c0), 0, nv * 16,
        kBufferWord3);

    // Ring slots: data and (wave-uniform) metadata: batch index, chunk, flags (1 valid, 2 first
    // batch of its chunk, 4 last; bits 8 up: the unit).
    u32x4 ring[kRing][kU];
    int s_b[kRing], s_c[kRing], s_flags[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) s_b[j] = s_c[j] = s_flags[j] = 0;

    // The wave's first P chunks of its own unit are wv, wv + W, ...; later ones come from the
    // unit's counter (which starts at W * P), requested one chunk ahead. Chunk ids only grow, so
    // every wave runs out of work.
    int cur_c = 0, cur_i = 0, cur_n = 0, taken = 0;
    uint32_t pending = 0u;
    auto take_chunk = [&]() -> int {
        int c;
        if (taken < P)
            c = wv + W * taken;
        else
            c = __builtin_amdgcn_readfirstlane(pending);
        ++taken;
        if (taken >= P && lane == 0)
            pending = __hip_atomic_fetch_add(&sh.next_chunk[iq], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
        return c < i_nch ? c : -1;
    };
    // Move the issue side to the unit with the most chunks left; false if none has any.
    const bool can_help = !(active && wv == 0);
    auto switch_unit = [&]() -> bool {
        if (!can_help) return false;
        int best = -1;
        uint32_t most = 0u;
        for (int u = 0; u < G; ++u) {
            const uint32_t n = __builtin_amdgcn_readfirstlane(sh.unit_nch[u]);
            const uint32_t next = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                &sh.next_chunk[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            const uint32_t left = next < n ? n - next : 0u;
            if (left > most) {
                most = left;
                best = u;
            }
        }
        if (best < 0) return false;
        iq = best;
        const int inv = __builtin_amdgcn_readfirstlane(sh.unit_nv[iq]);
        i_nb = (inv + kStep - 1) / kStep;
        i_nch = __builtin_amdgcn_readfirstlane(sh.unit_nch[iq]);
        rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<u32x4 *>(reinterpret_cast<const u32x4 *>(logits) +
                                (int64_t)uniform64((uint64_t)sh.unit_c0[iq])),
            0, inv * 16, kBufferWord3);
        taken = P;  // counter chunks only
        if (lane == 0)
            pending = __hip_atomic_fetch_add(&sh.next_chunk[iq], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
        return true;
    };
    // Load the next batch of the issue side's unit into slot j; once the unit has no chunks left
    // the slot stays empty and the issue side is stalled until the main loop moves it (empty
    // slots then follow every loaded one in processing order, so they are refilled in index
    // order).
    bool stalled = false;
    auto issue = [&](int j) {
        if (cur_i == cur_n) {
            const int c = stalled ? -1 : take_chunk();
            if (c < 0) {
                s_flags[j] = 0;
                cur_i = cur_n = 0;
                stalled = true;
                return;
            }
            cur_c = c;
            cur_i = 0;
            cur_n = min(CB, i_nb - c * CB);
        }
        const int b = cur_c * CB + cur_i;
        load_batch(rsrc, voff, b, ring[j]);
        s_b[j] = b;
        s_c[j] = cur_c;
        s_flags[j] = 1 | (cur_i == 0 ? 2 : 0) | (cur_i == cur_n - 1 ? 4 : 0) | (iq << 8);
        ++cur_i;
    };

    // Ragged ends of the unit belong to its wave 0 and are loaded up front.
    const bool rag_owner = active && wv == 0;
    float xh = -INFINITY, xt = -INFINITY;
    if (rag_owner) {
        if (ur.h0 + lane < ur.h1) xh = Elem<T>::load(logits, ur.h0 + lane);
        if (ur.t0 + lane < ur.t1) xt = Elem<T>::load(logits, ur.t0 + lane);
    }

#pragma unroll
    for (int j = 0; j < kRing; ++j) issue(j);

    // Seed: the lane maxima of the wave's first kSeedBatches batches (and its ragged ends).
    {
        float m = fmaxf(xh, xt);
#pragma unroll
        for (int j = 0; j < kSeedBatches; ++j) {
            if ((s_flags[j] & 1) && (s_flags[j] >> 8) == q) {
                float x[kU * EV], bmax;
                const int nvalid = min(kStep, nv - s_b[j] * kStep);
                if (nvalid < kStep)
                    unpack_batch<T, true>(ring[j], nvalid, lane, x, bmax);
                else
                    unpack_batch<T, false>(ring[j], kStep, lane, x, bmax);
                m = fmaxf(m, bmax);
            }
        }
        sh.seed_vals[wave * kWave + lane] = value_key(m);
    }

    WaveTopk w;
    w.top = 0ull;
    w.k = k;
    w.shared_tau = &sh.tau[q];
    w.qmask = (uint32_t)(kQueueSlots / G - 1);
    w.queue = sh.queue + q * (kQueueSlots / G);
    w.q_tail = &sh.q_tail[q];
    w.q_head = &sh.q_head[q];
    w.head = 0u;
    w.owner = active && wv == 0;  // the unit's oldest wave keeps its list
    w.home = true;
    set_tau(w, 0ull);
    // Threshold seed: the wave starts from the k-th largest of its own 64 lane maxima, then
    // publishes them; the unit's last wave to publish raises the unit threshold to the k-th
    // largest of all of them. Either has k real elements at or above it. The k-th largest of a
    // set of order-preserving value keys is the largest t with at least k keys at or above it,
    // found one bit at a time from the top with ballot counts. The gate waves (which reach this
    // point only after their tile) do not take part. A unit whose batches the first ones of its
    // waves nearly cover waits for the unit threshold before it offers anything (a short wait
    // that spares the owner most of the candidates); a longer unit does not wait, nor does one
    // with at most one batch per wave (the threshold would come after every batch is read).
    const bool has_tile =
        NTG > 0 && gate_tile_of(blockIdx.x, gridDim.x, gj.mtiles * gj.splits) >= 0;
    auto gate_slot = [&](int s) {
        return has_tile && s >= gate_first_wave<G>() && s < gate_first_wave<G>() + gate_waves<NTG>();
    };
    if (active) {
        const uint32_t mk = sh.seed_vals[wave * kWave + lane];
        uint32_t t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            if (__popcll(__ballot(mk >= c)) >= k) t = c;
        }
        raise_tau(w, (uint64_t)t << 32, lane);
        int n_seed = 0;  // the unit's waves that are not gate waves (at least its owner)
#pragma unroll
        for (int i = 0; i < W; ++i) n_seed += gate_slot(unit_slot<G>(q, i)) ? 0 : 1;
        const bool wait_seed = nb > W && nb <= W * kSeedBatches;
        if (!gate_slot(wave)) {
            uint32_t arrived = 0u;
            if (lane == 0)
                arrived = __hip_atomic_fetch_add(&sh.seeded[q], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
            if (__builtin_amdgcn_readfirstlane(arrived) == (uint32_t)n_seed - 1u) {
                // the last to arrive: every other seeding wave's maxima are in LDS. Up to four
                // waves: the k-th largest of all their maxima. More: the k-th largest of the 64
                // lane-wise maxima over the waves (each is a real element of a lane position no
                // other shares, so k of them at or above it are k real elements), one search
                // instead of one per wave.
                uint32_t u = 0u;
                if constexpr (W <= 4) {
                    uint32_t v[W];
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const int si = unit_slot<G>(q, i);
                        v[i] = gate_slot(si) ? 0u : sh.seed_vals[si * kWave + lane];
                    }
                    for (int bit = 31; bit >= 0; --bit) {
                        const uint32_t c = u | (1u << bit);
                        int n = 0;
#pragma unroll
                        for (int i = 0; i < W; ++i) n += __popcll(__ballot(v[i] >= c));
                        if (n >= k) u = c;
                    }
                } else {
                    uint32_t v = 0u;
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const int si = unit_slot<G>(q, i);
                        const uint32_t sv = gate_slot(si) ? 0u : sh.seed_vals[si * kWave + lane];
                        v = sv > v ? sv : v;
                    }
                    for (int bit = 31; bit >= 0; --bit) {
                        const uint32_t c = u | (1u << bit);
                        if (__popcll(__ballot(v >= c)) >= k) u = c;
                    }
                }
                raise_tau(w, (uint64_t)u << 32, lane);
                if (lane == 0)
                    __hip_atomic_store(&sh.seed_done[q], 1u, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            if (wait_seed) {  // every seeding wave gets here without waiting on anything
                while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                           &sh.seed_done[q], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) ==
                       0u)
                    __builtin_amdgcn_s_sleep(1);
                pull_tau(w);
            }
        }
    }
    // logsumexp reference, fixed for every unit: terms are 2^(x log2e). Rows whose terms leave
    // fp32's range go down the exact path at the end.
    constexpr float R = 0.f;

    // Ragged ends: their own sums, and candidates into this wave's list.
    if (rag_owner) {
        float rs = 0.f;
        if (ur.h0 + lane < ur.h1) rs += __builtin_amdgcn_exp2f(fmaf(xh, kLog2e, -R));
        if (ur.t0 + lane < ur.t1) rs += __builtin_amdgcn_exp2f(fmaf(xt, kLog2e, -R));
        sh.rag[q * kWave + lane] = rs;
        if (__ballot(!(rs <= kSumLimit)) != 0ull && lane == 0) sh.overflow[q] = 1u;
        u32x4 raw = Elem<T>::single(xh);
        offer_lanes<T, 1, 1>(w, &raw, __ballot(ur.h0 + lane < ur.h1 && xh >= w.tau_v), kWave,
                             (int32_t)(ur.h0 - ur.g0), 1, lane, stage);
        raw = Elem<T>::single(xt);
        offer_lanes<T, 1, 1>(w, &raw, __ballot(ur.t0 + lane < ur.t1 && xt >= w.tau_v), kWave,
                             (int32_t)(ur.t0 - ur.g0), 1, lane, stage);
    }

    // Main loop: process the oldest slot, then issue the next batch into it. The processing side
    // follows the slots' unit: when it changes, the wave joins the other unit's queue and
    // threshold (it never owns a list there).
    float csum = 0.f;
    int pq = q, p_nv = nv;
    int32_t idb0 = (int32_t)(ur.c0 * EV - ur.g0);
    uint64_t te_key = ~0ull;  // the threshold t_e was computed for
    float t_e = 0.f;
    bool more = true;
    while (more) {
        if (stalled && switch_unit()) {
            stalled = false;
#pragma unroll
            for (int j = 0; j < kRing; ++j)
                if (!(s_flags[j] & 1)) issue(j);
        }
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            if (!(s_flags[j] & 1)) {
                more = false;
                break;
            }
            if ((s_flags[j] >> 8) != pq) {
                pq = s_flags[j] >> 8;
                p_nv = __builtin_amdgcn_readfirstlane(sh.unit_nv[pq]);
                idb0 = __builtin_amdgcn_readfirstlane(sh.unit_idb0[pq]);
                w.shared_tau = &sh.tau[pq];
                w.queue = sh.queue + pq * (kQueueSlots / G);
                w.q_tail = &sh.q_tail[pq];
                w.q_head = &sh.q_head[pq];
                w.home = pq == q;
                set_tau(w, 0ull);
                te_key = ~0ull;
                // A helper offers nothing before the unit's seed is in its threshold (without
                // it every element would be a candidate). The unit's seeding waves reach the
                // seed without waiting on any other wave, so this wait ends.
                while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                           &sh.seed_done[pq], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) ==
                       0u)
                    __builtin_amdgcn_s_sleep(1);
            }
            if (w.owner) drain<false>(w, lane, false);
            pull_tau(w);
            if (w.tau_key != te_key) {  // the threshold's term, recomputed only when it moved
                te_key = w.tau_key;
                t_e = __builtin_amdgcn_exp2f(fmaf(w.tau_v, kLog2e, -R)) * kTermMargin;
            }
            if (s_flags[j] & 2) csum = 0.f;
            const int b = s_b[j];
            const int nvalid = min(kStep, p_nv - b * kStep);
            const int32_t id_base = idb0 + b * kStep * EV;
            if (nvalid < kStep)
                batch<T, true>(ring[j], nvalid, id_base, R, t_e, csum, w, lane, vstage, vid);
            else
                batch<T, false>(ring[j], kStep, id_base, R, t_e, csum, w, lane, vstage, vid);
            if (s_flags[j] & 4) {
                chunk_sums[((size_t)pq * nch_max + s_c[j]) * kWave + lane] = csum;
                if (__ballot(!(csum <= kSumLimit)) != 0ull && lane == 0) sh.overflow[pq] = 1u;
            }
            issue(j);
        }
    }

    // The owner keeps taking queued candidates until every wave of the workgroup has finished
    // (any of them may help its unit; none waits on anything but an owner's draining, so this
    // ends), which leaves little for the pass after the barrier.
    if (lane == 0)
        __hip_atomic_fetch_add(&sh.done_all, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (w.owner) {
        while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                   &sh.done_all, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) <
               (uint32_t)kWaves) {
            drain<true>(w, lane, false);
            __builtin_amdgcn_s_sleep(2);
        }
    }
    // Every wave is done, so every reserved queue slot is written and every chunk sum is in
    // LDS. Each wave of a unit adds a fixed range of its chunk sums (per lane, in chunk order);
    // the owner takes what is left in the queue.
    __syncthreads();
    float *psum = reinterpret_cast<float *>(sh.seed_vals);
    if (active) {
        float t = 0.f;
        int c = nch * wv / W;
        const int c1 = nch * (wv + 1) / W;
        for (; c + 8 <= c1; c += 8) {  // loads issued together, added in chunk order
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = csums[(c + i) * kWave + lane];
#pragma unroll
            for (int i = 0; i < 8; ++i) t += v[i];
        }
        for (; c < c1; ++c) t += csums[c * kWave + lane];
        psum[wave * kWave + lane] = t;
    }
    __syncthreads();
    if (!rag_owner) return;
    drain<true>(w, lane, true);
    // The unit's logsumexp: the waves' partial sums per lane in wave order, then the ragged
    // sums, then across lanes (fixed order); lse = (R + log2 total) ln 2.
    float ref = R, sum = 0.f;
    bool fast =
        __hip_atomic_load(&sh.overflow[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u;
    if (fast) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < W; ++i) t += psum[unit_slot<G>(q, i) * kWave + lane];
        t += sh.rag[q * kWave + lane];
        t = wave_sum(t);
        sum = t;
        fast = t >= kSumFloor;  // every term far below 1: too few significant bits left
    }
    if (!fast) {
        exact_pair<T>(logits, ur, lane, ref, sum);
    }
    const uint64_t top = w.top;
    if (S == 1) {
        const double lse = lse_value(ref, sum);
        if (lane < k) {
            cand_ids[unit * k + lane] = key_id(top);
            unary[unit * k + lane] = (float)((double)key_logit(top) - lse);
        }
        if (lane == 0 && lse_out) lse_out[unit] = (float)lse;
    } else {
        part_keys[unit * kWave + lane] = top;
        if (lane == 0) part_lse[unit] = make_float2(ref, sum);
    }
}

// Merge the S slice results of each row (one wave per row, slices in order). The slices' lists
// and pairs are loaded kMergeAhead at a time before any merge (one memory round trip for S up
// to that).
constexpr int kMergeAhead = 8;

__global__ __launch_bounds__(kWave) void topk_merge_kernel(
    int k, int S, const uint64_t *__restrict__ part_keys, const float2 *__restrict__ part_lse,
    int32_t *__restrict__ cand_ids, float *__restrict__ unary, float *__restrict__ lse_out) {
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    uint64_t acc = 0ull;
    float2 ls = make_float2(-INFINITY, 0.f);
    for (int s0 = 0; s0 < S; s0 += kMergeAhead) {
        uint64_t keys[kMergeAhead];
        float2 pr[kMergeAhead];
#pragma unroll
        for (int i = 0; i < kMergeAhead; ++i) {
            const int s = min(s0 + i, S - 1);  // in range; the repeats are not used
            keys[i] = part_keys[(row * S + s) * kWave + lane];
            pr[i] = part_lse[row * S + s];
        }
#pragma unroll
        for (int i = 0; i < kMergeAhead; ++i) {
            if (s0 + i >= S) break;
            acc = s0 + i == 0 ? keys[i] : wave_merge_desc(acc, keys[i], lane);
            lse_combine(ls.x, ls.y, pr[i].x, pr[i].y);
        }
    }
    const double lse = lse_value(ls.x, ls.y);
    if (lane < k) {
        cand_ids[row * k + lane] = key_id(acc);
        unary[row * k + lane] = (float)((double)key_logit(acc) - lse);
    }
    if (lane == 0 && lse_out) lse_out[row] = (float)lse;
}

size_t chunk_sum_bytes(int G, int nch_max) { return (size_t)G * nch_max * kWave * sizeof(float); }

// Gate tile width (MFMA tiles of 16 columns) when the top-k pass carries the gate; 0: it cannot.
int fused_gate_nt(int r) { return r <= 64 ? 4 : (r <= 128 ? 8 : 0); }

size_t gate_red_bytes(int nt) {
    return (nt == 4 ? gate_red_floats<4>() : nt == 8 ? gate_red_floats<8>() : 0) * sizeof(float);
}

int k1_grid(const TopkPlan &plan, int R) {
    return (R * plan.slices + plan.groups - 1) / plan.groups;
}

template <typename T, int G>
void launch_g(const TopkPlan &plan, int nt, dim3 grid, size_t lds, hipStream_t stream,
              const T *logits, int V, int k, int units, int32_t *cand_ids, float *unary,
              float *lse, uint64_t *part_keys, float2 *part_lse, const GateJob &gj) {
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, stream, logits, V, k, plan.slices,
                           units, plan.chunk_batches, plan.chunks, cand_ids, unary, lse,
                           part_keys, part_lse, gj);
    };
    if (nt == 4)
        go(topk_lse_kernel<T, G, 4>);
    else if (nt == 8)
        go(topk_lse_kernel<T, G, 8>);
    else
        go(topk_lse_kernel<T, G, 0>);
}

template <typename T>
hipError_t launch_k1(const TopkPlan &plan, const void *logits, int R, int V, int k,
                     int32_t *cand_ids, float *unary, float *lse, uint64_t *part_keys,
                     float2 *part_lse, int nt, const GateJob &gj, hipStream_t stream) {
    const int units = R * plan.slices;
    const dim3 grid((unsigned)k1_grid(plan, R));
    const size_t lds = chunk_sum_bytes(plan.groups, plan.chunks) + gate_red_bytes(nt);
    const T *x = static_cast<const T *>(logits);
    switch (plan.groups) {
    case 1: launch_g<T, 1>(plan, nt, grid, lds, stream, x, V, k, units, cand_ids, unary, lse, part_keys, part_lse, gj); break;
    case 2: launch_g<T, 2>(plan, nt, grid, lds, stream, x, V, k, units, cand_ids, unary, lse, part_keys, part_lse, gj); break;
    default: launch_g<T, 4>(plan, nt, grid, lds, stream, x, V, k, units, cand_ids, unary, lse, part_keys, part_lse, gj); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.slices == 1) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)R), dim3(kWave), 0, stream, k,
                       plan.slices, part_keys, part_lse, cand_ids, unary, lse);
    return hipGetLastError();
}

}  // namespace

TopkPlan plan_topk(int R, int V, int elem_bytes) {
    const int64_t EV = 16 / elem_bytes;
    const int64_t nvec_row = V / EV + 1;  // whole vectors of a row, rounded up
    const int64_t nb_row = (nvec_row + kStep - 1) / kStep;
    TopkPlan p;
    // Slices only for fewer than kSliceBelowRows rows (enough slices for a unit per
    // workgroup), and never below kMinBatchesPerWave batches per wave.
    int64_t s = 1;
    if (R < kSliceBelowRows) {
        s = (kTargetWorkgroups + R - 1) / R;
        const int64_t s_max = nb_row / ((int64_t)kWaves * kMinBatchesPerWave);
        if (s > s_max) s = s_max;
        if (s < 1) s = 1;
    }
    p.slices = (int)s;
    const int64_t units = (int64_t)R * p.slices;
    p.groups = 1;
    while (p.groups * 2 <= kMaxUnits &&
           (units + p.groups * 2 - 1) / (p.groups * 2) >= kTargetWorkgroups)
        p.groups *= 2;
    p.waves = kWaves / p.groups;
    const int64_t nb_unit = (nvec_row / p.slices + 1 + kStep - 1) / kStep;  // slices differ by <= 1
    p.chunk_batches = 1;
    for (;;) {
        p.chunks = (int)((nb_unit + p.chunk_batches - 1) / p.chunk_batches);
        if (p.chunks < 1) p.chunks = 1;
        if (chunk_sum_bytes(p.groups, p.chunks) <= kLdsBudget) break;
        p.chunk_batches *= 2;
    }
    return p;
}

size_t topk_workspace_bytes(const TopkPlan &p, int R) {
    if (p.slices <= 1) return 0;
    return (size_t)R * p.slices * (kWave * sizeof(uint64_t) + sizeof(float2));
}

uint32_t next_launch_epoch() {
    static std::atomic<uint32_t> launches{0};
    uint32_t e = launches.fetch_add(1, std::memory_order_relaxed) + 1u;
    return e == 0u ? 1u : e;  // after 2^32 launches it wraps (the kernel then re-bases by CAS)
}

size_t topk_pass_workspace_bytes(int R, int V, int elem_bytes) {
    SmallPlanInfo sp;
    if (plan_small(R, V, elem_bytes, sp)) return small_workspace_bytes(sp, R);
    return topk_workspace_bytes(plan_topk(R, V, elem_bytes), R);
}

int fused_gate_splits(int R, int V, int logits_dtype, int H, int r) {
    SmallPlanInfo sp;
    if (plan_small(R, V, logits_dtype == 0 ? 4 : 2, sp))
        return small_gate_nt(r) ? gate_splits(R, H, 1) : 0;  // gate tiles as extra workgroups
    const int nt = fused_gate_nt(r);
    if (nt == 0) return 0;
    // The plan (its chunks above all) is the one the pass has without a gate, so both give the
    // same logsumexp bit for bit; the gate rides along only where its tile parts fit beside the
    // chunk sums.
    const TopkPlan plan = plan_topk(R, V, logits_dtype == 0 ? 4 : 2);
    if (chunk_sum_bytes(plan.groups, plan.chunks) + gate_red_bytes(nt) > kLdsDynamicMax) return 0;
    // one tile per workgroup; the grid holds at least R / 8 >= mtiles workgroups
    const int mtiles = (R + 15) / 16;
    const int most = k1_grid(plan, R) / mtiles;
    const int s = gate_splits(R, H, 1);
    return s < most ? s : most;
}

hipError_t launch_topk_lse(const void *logits, int logits_dtype, int R, int V, int k,
                           int32_t *cand_ids, float *unary, float *lse, void *workspace,
                           hipStream_t stream, const FusedGate *gate) {
    SmallPlanInfo sp;
    if (plan_small(R, V, logits_dtype == 0 ? 4 : 2, sp))
        return launch_topk_small(sp, logits, logits_dtype, R, V, k, next_launch_epoch(), cand_ids,
                                 unary, lse, workspace, stream, gate);
    const int nt = gate ? fused_gate_nt(gate->r) : 0;
    if (gate && nt == 0) return hipErrorInvalidValue;
    const TopkPlan plan = plan_topk(R, V, logits_dtype == 0 ? 4 : 2);
    uint64_t *part_keys = static_cast<uint64_t *>(workspace);
    float2 *part_lse = reinterpret_cast<float2 *>(part_keys + (size_t)R * plan.slices * kWave);
    GateJob gj{};
    if (gate) {
        gj.hidden = static_cast<const uint16_t *>(gate->hidden);
        gj.W = static_cast<const uint16_t *>(gate->W_sel);
        gj.part = gate->part;
        gj.R = R;
        gj.H = gate->H;
        gj.r = gate->r;
        gj.mtiles = (R + 15) / 16;
        gj.splits = fused_gate_splits(R, V, logits_dtype, gate->H, gate->r);
    }
    if (logits_dtype == 0)
        return launch_k1<float>(plan, logits, R, V, k, cand_ids, unary, lse, part_keys, part_lse,
                                nt, gj, stream);
    return launch_k1<uint16_t>(plan, logits, R, V, k, cand_ids, unary, lse, part_keys, part_lse,
                               nt, gj, stream);
}

}  // namespace dflash2
