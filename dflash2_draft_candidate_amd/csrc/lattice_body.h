// The lattice of one sequence and the greedy walk over it, as device code (the lattice kernels in
// lattice.hip run it, one workgroup per sequence or per pass of positions).
//
// edges[b][p][i][j] = unary[b][p][j] + sum_d pred_cb[prev_i][d] * succ_cb[cand_j][d] * g[b][p][d]
// with prev_i = anchor_ids[b] at p = 0 and cand_ids[b][p-1][i] after. Source: "DFlash 2: Keep
// Drafting Parallel" (inco.ai blog), section "A Lightweight Path Selector", eq.
// S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>; "DFlash2 Lands in llama.cpp" (ramgpt.org), section
// "What llama.cpp Actually Builds for the Selector" (successor rows of the current candidates,
// predecessor rows of the previous ones, the hidden gate of the current position; the anchor is
// the first predecessor). The walk: j_0 = argmax_j edges[b][0][0][j], j_p = argmax_j
// edges[b][p][j_{p-1}][j], ties to the lowest j (same sources: greedy from the last verified
// token, best successor of the chosen predecessor).
//
// Per position the lattice is a small product E = (P * g) S^T with P, S the gathered [k, r]
// codebook rows: it runs on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation). The
// fp32 operand a = P * g is split into three bf16 values, a = a1 + a2 + a3 + O(2^-27 |a|) (each
// rounded to nearest from the exact remainder), and each part is multiplied exactly (bf16 x bf16
// fits fp32) by the bf16 codebook value: three MFMAs per step, with the operand as accurate as an
// fp32 product. fp32 codebooks are split the same way and the six part products down to 2^-18
// |a b| are kept (a1b1, a2b1, a1b2, a3b1, a2b2, a1b3; the rest are below 2^-27 |a b|). With only
// two parts the remainder (2^-18 |a|) is large enough to break the 1e-5 edge tolerance where few
// ranks carry large codebook values. A wave owns one position and one 16-row tile of predecessors
// (KT = ceil(k / 16) waves per position) and all KT column tiles. The rank is cut into chunks of
// 64: within a chunk, lane group g = lane / 16 holds ranks 16g .. 16g + 15 of its rows, and MFMA
// step t (of 2) takes ranks 16g + 8t .. 16g + 8t + 7 as its K slots 8g .. 8g + 7 (any assignment
// of ranks to K slots gives the same sum; this one lets every lane fetch its 16 ranks with
// 16-byte loads). The chain per position is two dependent global round trips: ids, unary and the
// gate partials, then the codebook rows.
//
// The walk rides in the same workgroup: one workgroup per sequence computes every position, each
// wave reduces its rows to the best successor best[p][i] (wave-level argmax over an
// order-preserving key, lowest j on ties), and the oldest wave chases j_p = best[p][j_{p-1}] with
// v_readlane, one pass of positions at a time. With p_min > 0 each row also gets its greedy
// confidence 1 / sum_j exp(e_j - max) ("DFlash2 Lands in llama.cpp", section "p_min Means
// Something Different Under DFlash2"), and the chase records where the drafted block ends.
// Without the walk, a workgroup takes one pass of one sequence.
//
// Invalid ids: a row whose predecessor or candidate id lies outside [0, V) is written as NaN
// (row 0 is read in its place). The walk then follows the stand-alone walk's rule: a NaN at
// j = 0 makes j = 0 the choice, a NaN elsewhere never wins.
#pragma once

#include "device_common.h"

namespace dflash2 {

constexpr int kLatWaves = 16;                 // waves per workgroup at most

// Waves per workgroup for KT tiles and codebook element size cb: 4 x 4 tiles per wave (and 2 x 2
// tiles of fp32 codebooks) hold too many registers for 16 waves.
constexpr int lat_waves(int kt, int cb) { return kt == 4 || (kt == 2 && cb == 4) ? 8 : kLatWaves; }
constexpr int kRankChunk = 64;                // ranks per chunk: 4 lane groups x 16 steps
constexpr int kMaxPasses = 4;                 // the walk rides along up to this many passes
constexpr int kMaxSplit = 8;                  // gate partials per row at most (split-K)
template <typename CB, int KT>
constexpr bool kPipelined = sizeof(CB) == 2 && KT == 1;  // codebook chunks loaded one ahead

// Loads of ids, unary and gate partials: COHERENT when other workgroups of the same launch wrote
// them (device-scope loads, which do not return a stale line of this XCD's L2).
template <bool COHERENT, typename T>
__device__ __forceinline__ T lat_load(const T *p) {
    if constexpr (COHERENT)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

// 16 consecutive codebook values of one row as raw 16-byte vectors.
template <typename CB>
struct Seg {
    static constexpr int EV = Elem<CB>::kPerVec;
    static constexpr int NV = 16 / EV;  // 2 (bf16) or 4 (fp32) vectors
    u32x4 v[NV];
};

// Ranks seg .. seg + 15 of `row` (zeros past nval). vec: whole 16-byte vectors in bounds.
template <typename CB>
__device__ __forceinline__ void load_seg(Seg<CB> &s, const CB *row, int seg, int nval, bool vec) {
    if (vec) {
#pragma unroll
        for (int q = 0; q < Seg<CB>::NV; ++q)
            s.v[q] = *reinterpret_cast<const u32x4 *>(row + seg + q * Seg<CB>::EV);
        return;
    }
    CB tmp[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) tmp[e] = e < nval ? row[seg + e] : CB(0);
#pragma unroll
    for (int q = 0; q < Seg<CB>::NV; ++q) s.v[q] = *reinterpret_cast<const u32x4 *>(tmp + q * Seg<CB>::EV);
}

// Ranks 8t .. 8t + 7 of a segment, widened to fp32.
template <typename CB>
__device__ __forceinline__ void widen_half(const Seg<CB> &s, int t, float *x) {
#pragma unroll
    for (int q = 0; q < Seg<CB>::NV / 2; ++q)
        Elem<CB>::unpack(s.v[t * (Seg<CB>::NV / 2) + q], x + q * Seg<CB>::EV);
}

// Part of the gate row of one position into LDS: gw[d] = sum over the ksplit partial rows
// (stride apart) of the value at base + d, added in split order from 0, for d = d0 + lane + 64 dd
// (dd < ND). Only the loads that are needed are issued (rank chunks that start below r, splits
// below ksplit: wave-uniform conditions; lanes past r read rank r - 1), all of them before any
// sum: one memory round trip for up to 128 ranks at any split count (KS >= ksplit). Every load a
// wave issues costs the CU's memory pipeline a slot, and sixteen waves share it.
template <int ND, int KS, bool COHERENT>
__device__ __forceinline__ void gate_row(const float *gpart, int ksplit, int64_t stride,
                                         int64_t base, int r, int rpad, int lane, float *gw,
                                         int d0 = 0) {
    float part[ND][KS];
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
        const bool live = d0 + kWave * dd < r;
        const int d = min(d0 + lane + kWave * dd, r - 1);
#pragma unroll
        for (int q = 0; q < KS; ++q)
            part[dd][q] = live && q < ksplit ? lat_load<COHERENT>(&gpart[q * stride + base + d])
                                             : 0.f;
    }
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < KS; ++q)
            if (q < ksplit) v += part[dd][q];
        const int d = d0 + lane + kWave * dd;
        if (d < rpad) gw[d] = d < r ? v : 0.f;
    }
}

// x = x1 + x2 + x3 + O(2^-27 |x|), each bf16 rounded to nearest (every remainder is exact in
// fp32), for N values (N / 8 fragments each).
template <int N>
__device__ __forceinline__ void split3_bf16(const float *x, bf16x8 *x1, bf16x8 *x2, bf16x8 *x3) {
#pragma unroll
    for (int s = 0; s < N; ++s) {
        const __bf16 h1 = (__bf16)x[s];
        const float r1 = x[s] - (float)h1;
        const __bf16 h2 = (__bf16)r1;
        x1[s / 8][s % 8] = h1;
        x2[s / 8][s % 8] = h2;
        x3[s / 8][s % 8] = (__bf16)(r1 - (float)h2);
    }
}

// Walk key of edge value e in column j < k: larger key = better successor; equal keys go to the
// lower j. A NaN at j = 0 beats everything, a NaN elsewhere loses to everything (key 0, as for
// the padding columns).
__device__ __forceinline__ uint32_t walk_key(float e, int j) {
    if (e != e) return j == 0 ? 0xFFFFFFFFu : 0u;
    return value_key(e);
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRor8, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRor4, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false));
    return v;
}

// LDS of the lattice of one sequence (besides the gate rows): each position's best successor
// rows, candidate ids and confidences, for two passes with the walk.
template <bool WALK>
struct LatShared {
    // per row, the best successor at each position of the pass (row-major: one row's sixteen
    // positions are one 16-byte word for the chase)
    alignas(16) uint8_t best_s[WALK ? 2 : 1][kWave][kLatWaves];
    int32_t cand_s[WALK ? 2 : 1][kLatWaves][kWave];
    alignas(16) float conf_s[WALK ? 2 : 1][kWave][kLatWaves];  // p_min: confidence of each row
};

// The lattice's inputs and outputs (B sequences of L positions).
template <typename CB>
struct LatArgs {
    const int32_t *cand_ids;  // [B, L, k]
    const float *unary;       // [B, L, k]
    const float *gpart;       // [ksplit][B * L][r]
    int ksplit;
    const CB *pred, *succ;    // [V, r]
    const int32_t *anchor;    // [B]
    int B, L, V, r, k, pp;    // pp positions per pass
    float *edges;             // [B, L, k, k]
    int32_t *path;            // [B, L] (walk)
    int32_t *path_idx;        // [B, L] or null
    float p_min;
    int32_t *draft_len;       // [B] or null
};

// The lattice of sequence b by the waves of one workgroup: with WALK every pass in turn and the
// walk (every wave of the workgroup calls this: it holds barriers; ONE: a single pass), else pass
// `pass_only`. pp
// positions per pass, KT waves per position; waves past pp * KT take no position. gsh: the gate
// rows, [pp * KT][rpad] floats.
template <typename CB, int KT, bool WALK, bool COHERENT, bool ONE = false>
__device__ void lattice_sequence(const LatArgs<CB> &a, int b, int pass_only, int wave, int lane,
                                 LatShared<WALK> &ls, float *gsh) {
    const int32_t *__restrict__ cand_ids = a.cand_ids;
    const float *__restrict__ unary = a.unary;
    const float *__restrict__ gpart = a.gpart;
    const int ksplit = a.ksplit;
    const CB *__restrict__ pred = a.pred;
    const CB *__restrict__ succ = a.succ;
    const int32_t *__restrict__ anchor = a.anchor;
    const int L = a.L, V = a.V, r = a.r, k = a.k, pp = a.pp;
    float *__restrict__ edges = a.edges;
    int32_t *__restrict__ path = a.path;
    int32_t *__restrict__ path_idx = a.path_idx;
    const float p_min = a.p_min;
    int32_t *__restrict__ draft_len = a.draft_len;
    auto &best_s = ls.best_s;
    auto &cand_s = ls.cand_s;
    auto &conf_s = ls.conf_s;
    int stop = L;  // p_min: the drafted block's length (chasing wave)

    const int pl = wave / KT, ti = wave % KT;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t R = (int64_t)a.B * L;
    const int rpad = (r + kRankChunk - 1) / kRankChunk * kRankChunk;
    float *gw = gsh + (size_t)wave * rpad;
    const bool vec = (r % Seg<CB>::EV) == 0;
    // (ONE: the caller knows the block is one pass, L <= pp. Around a loop whose trip count is
    // only known at run time the compiler hoists the body's invariant lane masks to the kernel's
    // start and keeps them in spilled registers: several hundred instructions before each wave's
    // first load, so that with four waves a SIMD the younger ones reached their loads
    // microseconds late.)
    const int passes = WALK && !ONE ? (L + pp - 1) / pp : 1;
    int prev = 0;  // walk: the chosen index at the previous position (the anchor's row is 0)

    for (int pass = 0; pass < passes; ++pass) {
        const int p0 = (WALK ? pass : pass_only) * pp;
        const int np = min(pp, L - p0);
        const int buf = WALK ? (pass & 1) : 0;
        if (pl < np) {
            const int p = p0 + pl;
            const int64_t row = (int64_t)b * L + p;
            // Round trip 1: ids, unary, gate partials (independent loads).
            const int i = 16 * ti + li;
            int32_t pid = 0;
            if (i < k) pid = (p == 0) ? anchor[b] : lat_load<COHERENT>(&cand_ids[(row - 1) * k + i]);
            int32_t cid[KT];
            float u[KT];
#pragma unroll
            for (int tj = 0; tj < KT; ++tj) {
                const int j = 16 * tj + li;
                cid[tj] = j < k ? lat_load<COHERENT>(&cand_ids[row * k + j]) : 0;
                u[tj] = j < k ? lat_load<COHERENT>(&unary[row * k + j]) : 0.f;
            }
            {
                const int64_t stride = R * r, base = row * r;
                // 128 ranks per round trip where the codebook chunks are pipelined, else 64
                constexpr int ND = kPipelined<CB, KT> ? 2 : 1;
                for (int d0 = 0; d0 < rpad; d0 += ND * kWave)
                    gate_row<ND, kMaxSplit, COHERENT>(gpart, ksplit, stride, base, r, rpad, lane, gw,
                                                      d0);
            }
            const bool pok = pid >= 0 && pid < V;
            const uint32_t prow_ok = (uint32_t)__ballot(pok) & 0xFFFFu;  // bit li: row 16ti+li
            bool cok[KT];
#pragma unroll
            for (int tj = 0; tj < KT; ++tj) cok[tj] = cid[tj] >= 0 && cid[tj] < V;
            const CB *prow = pred + (int64_t)(pok ? pid : 0) * r;
            const CB *srow[KT];
#pragma unroll
            for (int tj = 0; tj < KT; ++tj) srow[tj] = succ + (int64_t)(cok[tj] ? cid[tj] : 0) * r;
            // the gate row is in LDS (written by this wave's lanes; LDS is in order per wave)
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

            // Round trip 2: the codebook rows, per chunk of 64 ranks. bf16 codebooks and one column
            // tile: the next chunk's loads are issued before the current chunk's MFMA steps (two
            // chunks in flight); the other shapes have no registers to spare for that.
            f32x4 acc[KT];
#pragma unroll
            for (int tj = 0; tj < KT; ++tj) acc[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
            auto chunk_loads = [&](int c0, Seg<CB> &sa, Seg<CB> *sb) {
                const int seg = c0 + 16 * lg;
                const int nval = max(0, min(16, r - seg));
                const bool vseg = vec && nval == 16;
                load_seg<CB>(sa, prow, seg, nval, vseg);
#pragma unroll
                for (int tj = 0; tj < KT; ++tj) load_seg<CB>(sb[tj], srow[tj], seg, nval, vseg);
            };
            auto chunk_mfma = [&](int c0, const Seg<CB> &sa, const Seg<CB> *sb) {
                const int seg = c0 + 16 * lg;
                // one half of the 16 ranks at a time: its three bf16 parts, then every tile's MFMAs
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    float a[8];
                    widen_half<CB>(sa, t, a);
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float4 gq = *reinterpret_cast<const float4 *>(gw + seg + 8 * t + 4 * q);
                        a[4 * q] *= gq.x; a[4 * q + 1] *= gq.y; a[4 * q + 2] *= gq.z; a[4 * q + 3] *= gq.w;
                    }
                    bf16x8 a1[1], a2[1], a3[1];
                    split3_bf16<8>(a, a1, a2, a3);
#pragma unroll
                    for (int tj = 0; tj < KT; ++tj) {
                        if constexpr (sizeof(CB) == 2) {  // bf16 codebook: exact operand
                            const bf16x8 bv = __builtin_bit_cast(bf16x8, sb[tj].v[t]);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], bv, acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[0], bv, acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3[0], bv, acc[tj], 0, 0, 0);
                        } else {
                            // both operands split in three; the products kept are those down to
                            // 2^-18 of a b (the others are below 2^-27 |a b|)
                            float bv[8];
                            widen_half<CB>(sb[tj], t, bv);
                            bf16x8 b1[1], b2[1], b3[1];
                            split3_bf16<8>(bv, b1, b2, b3);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], b1[0], acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[0], b1[0], acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], b2[0], acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3[0], b1[0], acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[0], b2[0], acc[tj], 0, 0, 0);
                            acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[0], b3[0], acc[tj], 0, 0, 0);
                        }
                    }
                }
            };
            if constexpr (kPipelined<CB, KT>) {
                Seg<CB> sa0, sb0[KT], sa1, sb1[KT];
                chunk_loads(0, sa0, sb0);
                for (int c0 = 0; c0 < r; c0 += 2 * kRankChunk) {
                    const int c1 = c0 + kRankChunk;
                    if (c1 < r) chunk_loads(c1, sa1, sb1);
                    chunk_mfma(c0, sa0, sb0);
                    if (c1 < r) {
                        if (c1 + kRankChunk < r) chunk_loads(c1 + kRankChunk, sa0, sb0);
                        chunk_mfma(c1, sa1, sb1);
                    }
                }
            } else {
                for (int c0 = 0; c0 < r; c0 += kRankChunk) {
                    Seg<CB> sa, sb[KT];
                    chunk_loads(c0, sa, sb);
                    chunk_mfma(c0, sa, sb);
                }
            }

            // acc[tj][t]: row 16ti + 4lg + t, column 16tj + li.
            float *erow = edges + row * k * k;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int ii = 16 * ti + 4 * lg + t;
                const bool rok = (prow_ok >> (4 * lg + t)) & 1u;
                uint32_t key[KT];
                float ev[KT];
#pragma unroll
                for (int tj = 0; tj < KT; ++tj) {
                    const int j = 16 * tj + li;
                    float e = u[tj] + acc[tj][t];
                    if (!rok || !cok[tj]) e = __builtin_nanf("");
                    ev[tj] = e;
                    key[tj] = j < k ? walk_key(e, j) : 0u;
                    if (ii < k && j < k) erow[ii * k + j] = e;
                }
                if (WALK) {
                    // best successor of row ii: the largest key of the row (16 lanes x KT
                    // tiles), then the lowest column holding it
                    uint32_t m = key[0];
#pragma unroll
                    for (int tj = 1; tj < KT; ++tj) m = umax32(m, key[tj]);
                    m = row16_max(m);
                    int jb = -1;
#pragma unroll
                    for (int tj = KT - 1; tj >= 0; --tj) {
                        const uint32_t hits = (uint32_t)(__ballot(key[tj] == m) >> (16 * lg)) & 0xFFFFu;
                        if (hits) jb = 16 * tj + __builtin_ctz(hits);
                    }
                    if (li == 0 && ii < k) best_s[buf][ii][pl] = (uint8_t)jb;
                    if (p_min > 0.f) {
                        // confidence at the row's maximum: 1 / sum_j exp(e_j - max)
                        const float mv = key_value(m);
                        float z = 0.f;
#pragma unroll
                        for (int tj = 0; tj < KT; ++tj)
                            z += 16 * tj + li < k ? __builtin_amdgcn_exp2f((ev[tj] - mv) * kLog2e) : 0.f;
                        z = row16_sum(z);
                        if (li == 0 && ii < k) conf_s[buf][ii][pl] = 1.f / z;
                    }
                }
            }
            if (WALK) {
                if (ti == 0 && lg == 0) {
#pragma unroll
                    for (int tj = 0; tj < KT; ++tj)
                        if (16 * tj + li < k) cand_s[buf][pl][16 * tj + li] = cid[tj];
                }
            }
        }
        if (WALK) {
            // Every position of the pass has its best successors in LDS. The oldest wave chases
            // the pointers; the others go on with the next pass (the other buffer), and the pass
            // after that starts only once this wave has reached the next barrier.
            __syncthreads();
            if (wave == 0) {
                // best[q][i] for row i = lane, four positions per register (indices < 64 fit a
                // byte), and with p_min each row's confidence: the chase reads them with
                // v_readlane, so its dependent steps touch no memory. A row's entries are one
                // 16-byte LDS read (the bytes of positions past the pass are stale and never read).
                static_assert(kLatWaves == 16, "a row's best successors fill one 16-byte word");
                const int src = lane < k ? lane : 0;
                const u32x4 bw = *reinterpret_cast<const u32x4 *>(&best_s[buf][src][0]);
                const uint32_t bj[kLatWaves / 4] = {bw.x, bw.y, bw.z, bw.w};
                // Every step runs (no branch per step): past np the bytes are stale and only
                // steer v_readlane (which reads lane index & 63) until the loop ends; prev keeps
                // the step np - 1 choice for the next pass. The choice of step q (< 64) goes to
                // byte q of four wave-uniform words, which lane q reads at the end.
                uint32_t pj[kLatWaves / 4] = {0u, 0u, 0u, 0u};
                int cur = prev;
                if (p_min > 0.f) {
                    float cf[kLatWaves];
#pragma unroll
                    for (int g = 0; g < kLatWaves / 4; ++g) {
                        const f32x4 c4 = *reinterpret_cast<const f32x4 *>(&conf_s[buf][src][4 * g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) cf[4 * g + e] = c4[e];
                    }
#pragma unroll
                    for (int q = 0; q < kLatWaves; ++q) {
                        const float c = __uint_as_float(
                            __builtin_amdgcn_readlane(__float_as_uint(cf[q]), cur));
                        stop = (q < np && stop == L && c < p_min) ? p0 + q : stop;
                        const int j = (int)((__builtin_amdgcn_readlane(bj[q / 4], cur) >>
                                             (8 * (q % 4))) & 0xFFu);
                        pj[q / 4] |= (uint32_t)j << (8 * (q % 4));
                        prev = q == np - 1 ? j : prev;
                        cur = j;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < kLatWaves; ++q) {
                        const int j = (int)((__builtin_amdgcn_readlane(bj[q / 4], cur) >>
                                             (8 * (q % 4))) & 0xFFu);
                        pj[q / 4] |= (uint32_t)j << (8 * (q % 4));
                        prev = q == np - 1 ? j : prev;
                        cur = j;
                    }
                }
                const uint32_t pw = lane < 4 ? pj[0] : lane < 8 ? pj[1] : lane < 12 ? pj[2] : pj[3];
                const int out_j = (int)((pw >> (8 * (lane & 3))) & 0xFFu);
                if (lane < np) {
                    path[(int64_t)b * L + p0 + lane] = cand_s[buf][lane][out_j];
                    if (path_idx) path_idx[(int64_t)b * L + p0 + lane] = out_j;
                }
            }
        }
    }
    if (WALK && wave == 0 && lane == 0 && draft_len) draft_len[b] = stop;
}

}  // namespace dflash2
