// The C ABI (include/dflash2.h): host-side validation, workspace layout and launches.
// Nothing here allocates device memory or synchronises; all work goes to the caller's stream.
#include "dflash2.h"

#include <float.h>
#include <limits.h>

#include <mutex>

#include "kernels.h"

namespace {

using namespace dflash2;

constexpr size_t kAlign = 256;  // workspace sub-buffer alignment

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int dt) { return dt == DFLASH2_F32 || dt == DFLASH2_BF16; }

int hip_status(hipError_t e) { return e == hipSuccess ? DFLASH2_OK : DFLASH2_ERR_HIP; }

// Sizes shared by select and its stages; 0 = valid.
int check_rows(int R, int V, int k) {
    if (R < 1 || V < 1 || V > DFLASH2_MAX_V || k < 1 || k > DFLASH2_MAX_K || k > V)
        return DFLASH2_ERR_INVALID_ARG;
    return DFLASH2_OK;
}

int check_ptrs(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (!p) return DFLASH2_ERR_INVALID_ARG;
    for (const void *p : ptrs)
        if (!aligned16(p)) return DFLASH2_ERR_ALIGNMENT;
    return DFLASH2_OK;
}

int64_t rows_of(int B, int L) { return (int64_t)B * L; }

struct SelectLayout {
    size_t lse, gpart, topk, total;
};

// Workspace of dflash2_select: lse [R] | gate partials [splits][R][r] | K1 slice partials.
// (The fused gate uses at most gate_splits splits.)
SelectLayout select_layout(int R, int V, int H, int r, int logits_dtype, int act_dtype) {
    SelectLayout s;
    size_t off = 0;
    s.lse = off;
    off += round_up((size_t)R * sizeof(float));
    s.gpart = off;
    off += round_up((size_t)gate_splits(R, H, act_dtype) * R * r * sizeof(float));
    s.topk = off;
    off += round_up(topk_pass_workspace_bytes(R, V, logits_dtype == DFLASH2_F32 ? 4 : 2));
    s.total = off;
    return s;
}

// Host-side validation of dflash2_select_ex's arguments other than the workspace.
int check_select(const void *logits, int logits_dtype, const void *hidden, int act_dtype,
                 const void *W_sel, const void *pred_cb, const void *succ_cb, int cb_dtype,
                 const int32_t *anchor_ids, int B, int L, int V, int H, int r, int k,
                 float temperature, const float *uniforms, float p_min, const int32_t *cand_ids,
                 const float *unary, const float *edges, const int32_t *path,
                 const int32_t *draft_len) {
    if (B < 1 || L < 1 || H < 1 || r < 1 || r > DFLASH2_MAX_R || rows_of(B, L) > INT_MAX)
        return DFLASH2_ERR_INVALID_ARG;
    int rc = check_rows((int)rows_of(B, L), V, k);
    if (rc) return rc;
    if (!dtype_ok(logits_dtype) || !dtype_ok(act_dtype) || !dtype_ok(cb_dtype))
        return DFLASH2_ERR_INVALID_ARG;
    if ((rc = check_ptrs({logits, hidden, W_sel, pred_cb, succ_cb, anchor_ids, cand_ids, unary,
                          edges, path})))
        return rc;
    if (!(temperature >= 0.f) || !(temperature <= FLT_MAX) || p_min != p_min ||
        (temperature > 0.f && !uniforms))
        return DFLASH2_ERR_INVALID_ARG;
    if ((uniforms && !aligned16(uniforms)) || (draft_len && !aligned16(draft_len)))
        return DFLASH2_ERR_ALIGNMENT;
    return DFLASH2_OK;
}

// The allocation-free entry point's workspace: one array per GPU, part of the loaded code object.
// In host code `scratch` names a host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device is ever passed on.
static __device__ __align__(256) unsigned char scratch[DFLASH2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of each GPU's array, once found

// The current device's scratch array (found on the first call with that device current).
int current_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH2_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return DFLASH2_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DFLASH2_OK;
}

}  // namespace

extern "C" {

int dflash2_version(void) { return DFLASH2_ABI_VERSION; }

const char *dflash2_status_string(int status) {
    switch (status) {
    case DFLASH2_OK: return "ok";
    case DFLASH2_ERR_INVALID_ARG: return "invalid argument (size, dtype or NULL pointer)";
    case DFLASH2_ERR_UNSUPPORTED: return "unsupported request";
    case DFLASH2_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case DFLASH2_ERR_WORKSPACE: return "workspace missing or too small";
    case DFLASH2_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

size_t dflash2_topk_lse_workspace_bytes(int R, int V, int k, int logits_dtype) {
    if (check_rows(R, V, k) != DFLASH2_OK || !dtype_ok(logits_dtype)) return 0;
    return topk_pass_workspace_bytes(R, V, logits_dtype == DFLASH2_F32 ? 4 : 2);
}

int dflash2_topk_lse(const void *logits, int logits_dtype, int R, int V, int k, int32_t *cand_ids,
                     float *unary, float *lse, void *workspace, size_t workspace_bytes,
                     void *stream) {
    int rc = check_rows(R, V, k);
    if (rc) return rc;
    if (!dtype_ok(logits_dtype)) return DFLASH2_ERR_INVALID_ARG;
    if ((int64_t)R * V / V != R) return DFLASH2_ERR_INVALID_ARG;
    if ((rc = check_ptrs({logits, cand_ids, unary}))) return rc;
    if (lse && !aligned16(lse)) return DFLASH2_ERR_ALIGNMENT;
    const size_t need = dflash2_topk_lse_workspace_bytes(R, V, k, logits_dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return DFLASH2_ERR_WORKSPACE;
        if (!aligned16(workspace)) return DFLASH2_ERR_ALIGNMENT;
    }
    return hip_status(launch_topk_lse(logits, logits_dtype, R, V, k, cand_ids, unary, lse,
                                      workspace, static_cast<hipStream_t>(stream)));
}

size_t dflash2_gate_workspace_bytes(int R, int H, int r) {
    if (R < 1 || H < 1 || r < 1 || r > DFLASH2_MAX_R) return 0;
    return gate_workspace_bytes(R, H, r, DFLASH2_BF16);
}

int dflash2_gate(const void *hidden, const void *W_sel, int act_dtype, int R, int H, int r,
                 float *g, void *workspace, size_t workspace_bytes, void *stream) {
    if (R < 1 || H < 1 || r < 1 || r > DFLASH2_MAX_R || !dtype_ok(act_dtype))
        return DFLASH2_ERR_INVALID_ARG;
    int rc = check_ptrs({hidden, W_sel, g});
    if (rc) return rc;
    const size_t need = act_dtype == DFLASH2_BF16 ? dflash2_gate_workspace_bytes(R, H, r) : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return DFLASH2_ERR_WORKSPACE;
        if (!aligned16(workspace)) return DFLASH2_ERR_ALIGNMENT;
    }
    return hip_status(launch_gate(hidden, W_sel, act_dtype, R, H, r, g, workspace,
                                  static_cast<hipStream_t>(stream)));
}

int dflash2_lattice(const int32_t *cand_ids, const float *unary, const float *g,
                    const void *pred_cb, const void *succ_cb, int cb_dtype,
                    const int32_t *anchor_ids, int B, int L, int V, int r, int k, float *edges,
                    void *stream) {
    if (B < 1 || L < 1 || V < 1 || r < 1 || r > DFLASH2_MAX_R || k < 1 || k > DFLASH2_MAX_K ||
        !dtype_ok(cb_dtype) || rows_of(B, L) > INT_MAX)
        return DFLASH2_ERR_INVALID_ARG;
    int rc = check_ptrs({cand_ids, unary, g, pred_cb, succ_cb, anchor_ids, edges});
    if (rc) return rc;
    return hip_status(launch_lattice(cand_ids, unary, g, 1, pred_cb, succ_cb, cb_dtype, anchor_ids,
                                     B, L, V, r, k, edges, static_cast<hipStream_t>(stream)));
}

int dflash2_walk(const float *edges, const int32_t *cand_ids, int B, int L, int k, int32_t *path,
                 int32_t *path_idx, void *stream) {
    if (B < 1 || L < 1 || k < 1 || k > DFLASH2_MAX_K || rows_of(B, L) > INT_MAX)
        return DFLASH2_ERR_INVALID_ARG;
    int rc = check_ptrs({edges, cand_ids, path});
    if (rc) return rc;
    if (path_idx && !aligned16(path_idx)) return DFLASH2_ERR_ALIGNMENT;
    return hip_status(launch_walk(edges, cand_ids, B, L, k, path, path_idx,
                                  static_cast<hipStream_t>(stream)));
}

int dflash2_walk_ex(const float *edges, const int32_t *cand_ids, int B, int L, int k,
                    float temperature, const float *uniforms, float p_min, int32_t *path,
                    int32_t *path_idx, int32_t *draft_len, void *stream) {
    if (B < 1 || L < 1 || k < 1 || k > DFLASH2_MAX_K || rows_of(B, L) > INT_MAX ||
        !(temperature >= 0.f) || !(temperature <= FLT_MAX) || p_min != p_min)
        return DFLASH2_ERR_INVALID_ARG;
    if (temperature > 0.f && !uniforms) return DFLASH2_ERR_INVALID_ARG;
    int rc = check_ptrs({edges, cand_ids, path});
    if (rc) return rc;
    for (const void *p : {(const void *)uniforms, (const void *)path_idx, (const void *)draft_len})
        if (p && !aligned16(p)) return DFLASH2_ERR_ALIGNMENT;
    WalkMode mode;
    mode.temperature = temperature;
    mode.uniforms = temperature > 0.f ? uniforms : nullptr;
    mode.p_min = p_min;
    mode.draft_len = draft_len;
    return hip_status(launch_walk(edges, cand_ids, B, L, k, path, path_idx,
                                  static_cast<hipStream_t>(stream), &mode));
}

int dflash2_dynconv(const void *x, const void *base, const void *dyn, int dtype, int n_blocks,
                    int T, int C, int K, int group, void *y, void *stream) {
    if (n_blocks < 1 || T < 1 || C < 1 || K < 1 || K > DFLASH2_MAX_CONV_TAPS || group < 1 ||
        C % group != 0 || !dtype_ok(dtype) ||
        (int64_t)n_blocks * T * ((C + 255) / 256) > INT_MAX)  // one-dimensional grid
        return DFLASH2_ERR_INVALID_ARG;
    int rc = check_ptrs({x, base, dyn, y});
    if (rc) return rc;
    return hip_status(launch_dynconv(x, base, dyn, dtype, n_blocks, T, C, K, group, y,
                                     static_cast<hipStream_t>(stream)));
}

static bool lmhead_args_valid(int R, int H, int V, int k) {
    return R >= 1 && H >= 8 && H % 8 == 0 && V >= 1 && V <= DFLASH2_MAX_V && k >= 1 &&
           k <= DFLASH2_LMHEAD_MAX_K && k <= lmhead_max_k() && k <= V;
}

size_t dflash2_lmhead_topk_workspace_bytes(int R, int H, int V, int k) {
    if (!lmhead_args_valid(R, H, V, k) || R > DFLASH2_LMHEAD_MAX_ROWS) return 0;
    return lmhead_workspace_bytes(R, V);
}

int dflash2_lmhead_topk(const void *hidden, const void *W_lm, int R, int H, int V, int k,
                        int32_t *cand_ids, float *unary, float *lse, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (!lmhead_args_valid(R, H, V, k)) return DFLASH2_ERR_INVALID_ARG;
    if (R > DFLASH2_LMHEAD_MAX_ROWS) return DFLASH2_ERR_UNSUPPORTED;
    const size_t need = dflash2_lmhead_topk_workspace_bytes(R, H, V, k);
    int rc = check_ptrs({hidden, W_lm, cand_ids, unary});
    if (rc) return rc;
    if (lse && !aligned16(lse)) return DFLASH2_ERR_ALIGNMENT;
    if (!workspace || workspace_bytes < need) return DFLASH2_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DFLASH2_ERR_ALIGNMENT;
    return hip_status(launch_lmhead_topk(hidden, W_lm, R, H, V, k, cand_ids, unary, lse,
                                         workspace, static_cast<hipStream_t>(stream)));
}

size_t dflash2_workspace_bytes(int B, int L, int V, int H, int r, int k) {
    if (B < 1 || L < 1 || H < 1 || r < 1 || r > DFLASH2_MAX_R || rows_of(B, L) > INT_MAX ||
        check_rows((int)rows_of(B, L), V, k) != DFLASH2_OK)
        return 0;
    const int R = (int)rows_of(B, L);
    size_t most = 0;
    for (int ld = DFLASH2_F32; ld <= DFLASH2_BF16; ++ld)
        for (int ad = DFLASH2_F32; ad <= DFLASH2_BF16; ++ad) {
            const size_t t = select_layout(R, V, H, r, ld, ad).total;
            most = t > most ? t : most;
        }
    return most;
}

int dflash2_select_ex(const void *logits, int logits_dtype, const void *hidden, int act_dtype,
                      const void *W_sel, const void *pred_cb, const void *succ_cb, int cb_dtype,
                      const int32_t *anchor_ids, int B, int L, int V, int H, int r, int k,
                      float temperature, const float *uniforms, float p_min, int32_t *cand_ids,
                      float *unary, float *edges, int32_t *path, int32_t *draft_len,
                      void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_select(logits, logits_dtype, hidden, act_dtype, W_sel, pred_cb, succ_cb,
                          cb_dtype, anchor_ids, B, L, V, H, r, k, temperature, uniforms, p_min,
                          cand_ids, unary, edges, path, draft_len);
    if (rc) return rc;
    const int R = (int)rows_of(B, L);
    const size_t need = dflash2_workspace_bytes(B, L, V, H, r, k);
    if (!workspace || workspace_bytes < need) return DFLASH2_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DFLASH2_ERR_ALIGNMENT;

    const SelectLayout lay = select_layout(R, V, H, r, logits_dtype, act_dtype);
    char *ws = static_cast<char *>(workspace);
    float *lse = reinterpret_cast<float *>(ws + lay.lse);
    float *gpart = reinterpret_cast<float *>(ws + lay.gpart);
    hipStream_t s = static_cast<hipStream_t>(stream);

    // bf16 activations: the top-k pass carries the gate product (r <= 128); otherwise the gate
    // kernel runs on its own.
    const int fused = act_dtype == DFLASH2_BF16 ? fused_gate_splits(R, V, logits_dtype, H, r) : 0;
    hipError_t e;
    int ksplit;
    if (fused > 0) {
        const FusedGate fg{hidden, W_sel, H, r, gpart};
        e = launch_topk_lse(logits, logits_dtype, R, V, k, cand_ids, unary, lse, ws + lay.topk, s,
                            &fg);
        ksplit = fused;
    } else {
        e = launch_topk_lse(logits, logits_dtype, R, V, k, cand_ids, unary, lse, ws + lay.topk, s);
        if (e == hipSuccess) e = launch_gate_partials(hidden, W_sel, act_dtype, R, H, r, gpart, s);
        ksplit = gate_splits(R, H, act_dtype);
    }
    if (e != hipSuccess) return hip_status(e);
    // Short blocks, greedy: lattice and walk in one kernel (one workgroup per sequence). Long
    // blocks spread the lattice over more workgroups, and sampling runs in the walk kernel.
    if (temperature == 0.f && lattice_walk_fits(L, k, cb_dtype))
        return hip_status(launch_lattice_walk(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb,
                                              cb_dtype, anchor_ids, B, L, V, r, k, edges, path,
                                              nullptr, p_min, draft_len, s));
    e = launch_lattice(cand_ids, unary, gpart, ksplit, pred_cb, succ_cb, cb_dtype, anchor_ids, B,
                       L, V, r, k, edges, s);
    WalkMode mode;
    mode.temperature = temperature;
    mode.uniforms = temperature > 0.f ? uniforms : nullptr;
    mode.p_min = p_min;
    mode.draft_len = draft_len;
    if (e == hipSuccess) e = launch_walk(edges, cand_ids, B, L, k, path, nullptr, s, &mode);
    return hip_status(e);
}

int dflash2_select(const void *logits, int logits_dtype, const void *hidden, int act_dtype,
                   const void *W_sel, const void *pred_cb, const void *succ_cb, int cb_dtype,
                   const int32_t *anchor_ids, int B, int L, int V, int H, int r, int k,
                   int32_t *cand_ids, float *unary, float *edges, int32_t *path, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return dflash2_select_ex(logits, logits_dtype, hidden, act_dtype, W_sel, pred_cb, succ_cb,
                             cb_dtype, anchor_ids, B, L, V, H, r, k, 0.f, nullptr, 0.f, cand_ids,
                             unary, edges, path, nullptr, workspace, workspace_bytes, stream);
}

int dflash2_select_noalloc(const void *logits, int logits_dtype, const void *hidden,
                           int act_dtype, const void *W_sel, const void *pred_cb,
                           const void *succ_cb, int cb_dtype, const int32_t *anchor_ids, int B,
                           int L, int V, int H, int r, int k, int32_t *cand_ids, float *unary,
                           float *edges, int32_t *path, void *stream) {
    // every argument is checked before the array is looked up
    int rc = check_select(logits, logits_dtype, hidden, act_dtype, W_sel, pred_cb, succ_cb,
                          cb_dtype, anchor_ids, B, L, V, H, r, k, 0.f, nullptr, 0.f, cand_ids,
                          unary, edges, path, nullptr);
    if (rc) return rc;
    if (dflash2_workspace_bytes(B, L, V, H, r, k) > DFLASH2_NOALLOC_SCRATCH_BYTES)
        return DFLASH2_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((rc = current_scratch(&ws)) != DFLASH2_OK) return rc;
    return dflash2_select_ex(logits, logits_dtype, hidden, act_dtype, W_sel, pred_cb, succ_cb,
                             cb_dtype, anchor_ids, B, L, V, H, r, k, 0.f, nullptr, 0.f, cand_ids,
                             unary, edges, path, nullptr, ws, DFLASH2_NOALLOC_SCRATCH_BYTES,
                             stream);
}

}  // extern "C"
