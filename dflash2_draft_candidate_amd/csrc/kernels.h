// Internal launch interface between the C ABI (dflash2_abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash2 {

// ---- K1: top-k + logsumexp -----------------------------------------------------------------
struct TopkPlan {
    int waves;          // waves per (row, slice) unit
    int slices;         // slices per row; > 1 adds a merge kernel and needs workspace
    int groups;         // units per workgroup
    int chunk_batches;  // batches per chunk handed to a wave
    int chunks;         // chunks per unit (at most)
};
TopkPlan plan_topk(int R, int V, int elem_bytes);
size_t topk_workspace_bytes(const TopkPlan &plan, int R);
// The gate product carried by the top-k pass (bf16 hidden and W_sel, r <= 128): it writes
// fused_gate_splits(...) partial products [splits][R][r] floats to `part`.
struct FusedGate {
    const void *hidden;
    const void *W_sel;
    int H, r;
    float *part;
};
// Splits of the fused gate for these sizes; 0 if the pass cannot carry the gate (r > 128).
int fused_gate_splits(int R, int V, int logits_dtype, int H, int r);
// Workspace of the top-k pass for these sizes (whichever kernel launch_topk_lse picks).
size_t topk_pass_workspace_bytes(int R, int V, int elem_bytes);
hipError_t launch_topk_lse(const void *logits, int logits_dtype, int R, int V, int k,
                           int32_t *cand_ids, float *unary, float *lse, void *workspace,
                           hipStream_t stream, const FusedGate *gate = nullptr);

// The top-k pass for rows too few to fill the chip (topk_small.hip): `slices` workgroups per
// row, one load round each, slices merged in the kernel through per-row arrival counters.
struct SmallPlanInfo {
    int slices;
};
bool plan_small(int R, int V, int elem_bytes, SmallPlanInfo &plan);
size_t small_workspace_bytes(const SmallPlanInfo &plan, int R);
int small_gate_nt(int r);  // gate tile width it carries for rank r (0: r too large)
hipError_t launch_topk_small(const SmallPlanInfo &plan, const void *logits, int logits_dtype,
                             int R, int V, int k, uint32_t epoch, int32_t *cand_ids, float *unary,
                             float *lse, void *workspace, hipStream_t stream,
                             const FusedGate *gate);
// The arrival counters' epoch for one launch: a process-wide launch count (never 0), so epochs grow
// from launch to launch until the count wraps.
uint32_t next_launch_epoch();

// ---- K2: gate GEMM ---------------------------------------------------------------------------
// bf16 runs as `gate_splits` partial products over ranges of H, [splits][R][r] floats;
// fp32 runs as one split. launch_gate_partials writes the partials (one split = g itself);
// launch_gate also sums them into g (workspace: gate_workspace_bytes).
int gate_splits(int R, int H, int act_dtype);
size_t gate_workspace_bytes(int R, int H, int r, int act_dtype);
hipError_t launch_gate_partials(const void *hidden, const void *W_sel, int act_dtype, int R,
                                int H, int r, float *part, hipStream_t stream);
hipError_t launch_gate(const void *hidden, const void *W_sel, int act_dtype, int R, int H, int r,
                       float *g, void *workspace, hipStream_t stream);

// ---- K3: lattice -----------------------------------------------------------------------------
// gpart: the gate as `ksplit` partial rows [ksplit][B*L][r], summed in split order.
hipError_t launch_lattice(const int32_t *cand_ids, const float *unary, const float *gpart,
                          int ksplit, const void *pred_cb, const void *succ_cb, int cb_dtype,
                          const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                          float *edges, hipStream_t stream);
// The lattice with the greedy walk in the same kernel (one workgroup per sequence); for blocks
// where lattice_walk_fits(L, k, cb_dtype). path_idx may be null.
bool lattice_walk_fits(int L, int k, int cb_dtype);
hipError_t launch_lattice_walk(const int32_t *cand_ids, const float *unary, const float *gpart,
                               int ksplit, const void *pred_cb, const void *succ_cb, int cb_dtype,
                               const int32_t *anchor_ids, int B, int L, int V, int r, int k,
                               float *edges, int32_t *path, int32_t *path_idx, float p_min,
                               int32_t *draft_len, hipStream_t stream);

// ---- K4: walk --------------------------------------------------------------------------------
// The walk's modes: temperature 0 is greedy; > 0 draws by inverse CDF from uniforms [B, L];
// p_min > 0 writes the early-stop block length to draft_len [B] (may be null).
struct WalkMode {
    float temperature = 0.f;
    const float *uniforms = nullptr;
    float p_min = 0.f;
    int32_t *draft_len = nullptr;
};
hipError_t launch_walk(const float *edges, const int32_t *cand_ids, int B, int L, int k,
                       int32_t *path, int32_t *path_idx, hipStream_t stream,
                       const WalkMode *mode = nullptr);

// ---- LM-head product with the top-k pass in its epilogue -------------------------------------
// hidden [R, H] and W_lm [V, H] bf16 (H % 8 == 0), k <= lmhead_max_k(); workspace:
// lmhead_workspace_bytes(R, V) bytes of range partials.
int lmhead_max_k();
size_t lmhead_workspace_bytes(int R, int V);
hipError_t launch_lmhead_topk(const void *hidden, const void *W_lm, int R, int H, int V, int k,
                              int32_t *cand_ids, float *unary, float *lse, void *workspace,
                              hipStream_t stream);

// ---- grouped dynamic depthwise convolution of the draft blocks ------------------------------
hipError_t launch_dynconv(const void *x, const void *base, const void *dyn, int dtype, int nb,
                          int Tn, int C, int K, int G, void *y, hipStream_t stream);

}  // namespace dflash2
