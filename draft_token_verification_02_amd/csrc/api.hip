// C ABI of the verification step (declared in include/specverify.h):
// argument validation, workspace carving and kernel launches on the
// caller's stream.  No allocation, no synchronisation, no state.

#include <algorithm>
#include <cstring>
#include <mutex>

#include "sv_common.h"

namespace sv {
int lmhead_grid(int V);
hipError_t launch_lmhead_tiled(const uint16_t* htile, const uint16_t* W, bool w_tiled, int R,
                               int d, int V, float* logits, float* part_max, float* part_sum,
                               int32_t* part_arg, int NPs, int32_t* counters, int n_counters,
                               hipStream_t stream);
hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, bool w_tiled, int R, int d,
                         int V, float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                         int NPs, int grid, int32_t* counters, int n_counters, hipStream_t stream);
size_t tiled_w_bytes(int V, int d);
hipError_t launch_tile_rows(const uint16_t* W, int V, int d, uint16_t* Wt, hipStream_t stream);
hipError_t launch_greedy(const float* part_max, const int32_t* part_arg, int NP, int NPs, int B,
                         int gamma, int V, const int32_t* draft, int32_t* out_tokens,
                         int32_t* n_accepted, int32_t* target_tokens, int32_t* status,
                         hipStream_t stream);
hipError_t launch_accept_draw(const float* logits, const float* part_max, const float* part_sum,
                              int NP, int NPs, int B, int gamma, int V, const int32_t* draft,
                              const float* q, const int32_t* q_idx, int K, const float* uniforms,
                              int NC, const ChunkSums& cs, int32_t* counters,
                              float* row_max, float* row_sum, int32_t* out_tokens,
                              int32_t* n_accepted, int32_t* status, hipStream_t stream);
hipError_t launch_sparse_head(const uint16_t* h, const uint16_t* W, const uint16_t* cent,
                              const int32_t* members, int N, int d, int V, int C, int M, int k,
                              int32_t* q_ids, float* q_vals, int32_t* clusters, void* ws,
                              hipStream_t stream);
hipError_t launch_tree(const float* logits, const float* part_max, const float* part_sum, int NP,
                       int NPs, int B, int V, const TreeTopo& tp, int rounds,
                       const int32_t* tokens, const float* q, const float* uniforms, int NC,
                       const ChunkSums& cs, float* row_max, float* row_sum, void* state,
                       int32_t* counters, int32_t* out_tokens, int32_t* n_accepted,
                       int32_t* path_nodes, int32_t* status, hipStream_t stream);
}  // namespace sv

namespace {

bool w_shape_ok(int V, int d) { return d >= 8 && d <= 65536 && d % 8 == 0 && V >= 1 && V <= (1 << 28); }

bool layout_ok(int32_t l) { return l == SV_W_ROWS || l == SV_W_TILED; }

bool dims_ok(sv_dims d) {
    if (!(d.B >= 1 && d.B <= (1 << 20) && d.gamma >= 1 && d.gamma <= SV_MAX_GAMMA &&
          w_shape_ok(d.V, d.d) && layout_ok(d.w_layout)))
        return false;
    // the draw's chunk-sum grid has one workgroup per (sequence, chunk)
    const int64_t chunks = (d.V + sv::kDrawChunk - 1) / sv::kDrawChunk;
    return (int64_t)d.B * chunks <= INT32_MAX;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Softmax partials per row that stage 1 wrote for these dims.
int lmhead_partials(int R, int V) {
    return sv::lmhead_use_tiled(R, V) ? sv::lmhead_tiled_partials(V) : sv::lmhead_grid(V);
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

sv_status check_workspace(const void* ws, size_t bytes, sv_dims dims) {
    if (!ws) return SV_ERR_NULL;
    if (!aligned(ws, 256)) return SV_ERR_ALIGN;
    if (bytes < sv_workspace_bytes(dims)) return SV_ERR_WORKSPACE;
    return SV_OK;
}

// keep_logits = false (greedy verification) writes only the partials;
// with_argmax = false leaves out the greedy candidates (part_arg), which only
// greedy verification reads.
sv_status stage1(const uint16_t* hidden, const uint16_t* W, sv_dims dims, void* ws, hipStream_t s,
                 bool keep_logits = true, bool with_argmax = true) {
    const sv::Layout L = sv::make_layout(dims.B, dims.gamma, dims.d, dims.V);
    float* logits = keep_logits ? at<float>(ws, L.logits) : nullptr;
    int32_t* part_arg = with_argmax ? at<int32_t>(ws, L.part_arg) : nullptr;
    const bool w_tiled = dims.w_layout == SV_W_TILED;
    hipError_t e;
    if (sv::lmhead_use_tiled(L.R, dims.V)) {
        // the many-row GEMM reads the hidden rows tiled as well: a copy in
        // the workspace, made here (R d bf16 read and written once)
        uint16_t* htile = at<uint16_t>(ws, L.htile);
        e = sv::launch_tile_rows(hidden, L.R, dims.d, htile, s);
        if (e == hipSuccess)
            e = sv::launch_lmhead_tiled(htile, W, w_tiled, L.R, dims.d, dims.V, logits,
                                    at<float>(ws, L.part_max), at<float>(ws, L.part_sum),
                                    part_arg, L.NPs,
                                    at<int32_t>(ws, L.counters), dims.B * sv::kCounterStride, s);
    } else {
        e = sv::launch_lmhead(hidden, W, w_tiled, L.R, dims.d, dims.V, logits,
                              at<float>(ws, L.part_max), at<float>(ws, L.part_sum),
                              part_arg, L.NPs, sv::lmhead_grid(dims.V),
                              at<int32_t>(ws, L.counters), dims.B * sv::kCounterStride, s);
    }
    return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status stage2_greedy(const int32_t* draft, sv_dims dims, int32_t* out_tokens,
                        int32_t* n_accepted, int32_t* target_tokens, void* ws, hipStream_t s) {
    const sv::Layout L = sv::make_layout(dims.B, dims.gamma, dims.d, dims.V);
    hipError_t e = sv::launch_greedy(at<float>(ws, L.part_max), at<int32_t>(ws, L.part_arg),
                                     lmhead_partials(L.R, dims.V), L.NPs, dims.B, dims.gamma,
                                     dims.V, draft, out_tokens, n_accepted, target_tokens,
                                     at<int32_t>(ws, L.status), s);
    return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv::ChunkSums chunk_sums(void* ws, const sv::Layout& L) {
    return {at<double>(ws, L.csum), at<double>(ws, L.psum), at<double>(ws, L.cwave),
            at<double>(ws, L.pwave)};
}

// q_idx == nullptr: dense q [B][gamma][V]; otherwise sparse q with K entries per row.
sv_status stage2(const int32_t* draft, const float* q, const int32_t* q_idx, int K,
                 const float* uniforms, sv_dims dims, int32_t* out_tokens, int32_t* n_accepted,
                 void* ws, hipStream_t s) {
    const sv::Layout L = sv::make_layout(dims.B, dims.gamma, dims.d, dims.V);
    hipError_t e = sv::launch_accept_draw(
        at<float>(ws, L.logits), at<float>(ws, L.part_max), at<float>(ws, L.part_sum),
        lmhead_partials(L.R, dims.V), L.NPs, dims.B, dims.gamma, dims.V, draft, q, q_idx, K,
        uniforms, L.NC, chunk_sums(ws, L), at<int32_t>(ws, L.counters),
        at<float>(ws, L.row_max), at<float>(ws, L.row_sum),
        out_tokens, n_accepted, at<int32_t>(ws, L.status), s);
    return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status check_stage1(const uint16_t* hidden, const uint16_t* W, sv_dims dims, const void* ws,
                       size_t bytes) {
    if (!dims_ok(dims)) return SV_ERR_DIMS;
    if (!hidden || !W) return SV_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(W, 16)) return SV_ERR_ALIGN;
    return check_workspace(ws, bytes, dims);
}

sv_status check_stage2(const int32_t* draft, const float* q, const float* uniforms, sv_dims dims,
                       const int32_t* out_tokens, const int32_t* n_accepted, const void* ws,
                       size_t bytes) {
    if (!dims_ok(dims)) return SV_ERR_DIMS;
    if (!draft || !q || !uniforms || !out_tokens || !n_accepted) return SV_ERR_NULL;
    if (!aligned(q, 16) || !aligned(draft, 4) || !aligned(uniforms, 4) || !aligned(out_tokens, 4) ||
        !aligned(n_accepted, 4))
        return SV_ERR_ALIGN;
    return check_workspace(ws, bytes, dims);
}

sv_status check_stage2_sparse(const int32_t* draft, const int32_t* q_ids, const float* q_vals,
                              int32_t K, const float* uniforms, sv_dims dims,
                              const int32_t* out_tokens, const int32_t* n_accepted, const void* ws,
                              size_t bytes) {
    if (!dims_ok(dims) || K < 1 || K > (1 << 24)) return SV_ERR_DIMS;
    if (!draft || !q_ids || !q_vals || !uniforms || !out_tokens || !n_accepted) return SV_ERR_NULL;
    if (!aligned(q_ids, 16) || !aligned(q_vals, 16) || !aligned(draft, 4) || !aligned(uniforms, 4) ||
        !aligned(out_tokens, 4) || !aligned(n_accepted, 4))
        return SV_ERR_ALIGN;
    return check_workspace(ws, bytes, dims);
}

bool head_dims_ok(sv_head_dims d) {
    return d.N >= 1 && d.N <= 65535 && d.d >= 8 && d.d <= 65536 && d.d % 8 == 0 && d.V >= 1 &&
           d.V <= (1 << 28) && d.C >= 1 && d.C <= SV_HEAD_MAX_CLUSTERS && d.M >= 1 && d.k >= 1 &&
           d.k <= d.C && (int64_t)d.k * d.M <= (1 << 24);
}

bool tree_dims_ok(sv_dims d) {
    if (!(d.B >= 1 && d.B <= (1 << 20) && d.gamma >= 1 && d.gamma <= SV_MAX_TREE_NODES &&
          w_shape_ok(d.V, d.d) && layout_ok(d.w_layout)))
        return false;
    const int64_t chunks = (d.V + sv::kDrawChunk - 1) / sv::kDrawChunk;
    return (int64_t)d.B * chunks <= INT32_MAX;
}

// The most residual sums one walk from node v can need, plus its draw: a
// first child is tested against p; each rejection before the last child
// needs a sum to test the next one; the draw needs one.
int tree_rounds(const sv::TreeTopo& tp, int v) {
    const int row = v + 1;
    int t = tp.first_child[row];
    if (t < 0) return 1;
    int best = 0, j = 0;
    for (; t >= 0; t = tp.next_sibling[t], ++j) best = std::max(best, j + tree_rounds(tp, t));
    return std::max(best, j);                   // j children, all rejected
}

// Validates parent[] and builds the kernels' view of the topology.
bool build_topology(const int32_t* parent, int T, sv::TreeTopo* tp, int* rounds) {
    if (!parent || T < 1 || T > SV_MAX_TREE_NODES) return false;
    tp->T = T;
    for (int r = 0; r <= T; ++r) { tp->first_child[r] = -1; tp->qslot[r] = -1; }
    int depth[SV_MAX_TREE_NODES];
    int last_child[SV_MAX_TREE_NODES + 1];
    for (int r = 0; r <= T; ++r) last_child[r] = -1;
    tp->D = 0;
    for (int t = 0; t < T; ++t) {
        const int a = parent[t];
        if (a < -1 || a >= t) return false;
        depth[t] = a < 0 ? 1 : depth[a] + 1;
        tp->D = std::max(tp->D, depth[t]);
        tp->next_sibling[t] = -1;
        if (last_child[a + 1] < 0) tp->first_child[a + 1] = (int8_t)t;
        else tp->next_sibling[last_child[a + 1]] = (int8_t)t;
        last_child[a + 1] = t;
    }
    tp->P = 0;
    for (int r = 0; r <= T; ++r)
        if (tp->first_child[r] >= 0) tp->qslot[r] = (int8_t)tp->P++;
    if (rounds) *rounds = tree_rounds(*tp, -1);
    return true;
}

sv_status check_greedy(const int32_t* draft, sv_dims dims, const int32_t* out_tokens,
                       const int32_t* n_accepted, const int32_t* target_tokens, const void* ws,
                       size_t bytes) {
    if (!dims_ok(dims)) return SV_ERR_DIMS;
    if (!draft || !out_tokens || !n_accepted) return SV_ERR_NULL;
    if (!aligned(draft, 4) || !aligned(out_tokens, 4) || !aligned(n_accepted, 4) ||
        !aligned(target_tokens, 4))
        return SV_ERR_ALIGN;
    return check_workspace(ws, bytes, dims);
}

// Workspace of spec_verify_static: a file-scope device array, which every
// device the library runs on holds from module load until the process ends.
// In host code its name only stands in for it; its address on a device comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address goes to the kernels.
constexpr size_t kStaticScratchBytes = SV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of `scratch` on the current device.
sv_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_DEVICE;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return SV_ERR_DEVICE;
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

}  // namespace

extern "C" {

int32_t sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_string(sv_status status) {
    // A C caller may pass any int: read the argument's bytes as one rather
    // than loading an enum value outside the enum's range.
    int code;
    std::memcpy(&code, &status, sizeof code);
    switch (code) {
        case SV_OK: return "SV_OK";
        case SV_ERR_NULL: return "SV_ERR_NULL: a required pointer is NULL";
        case SV_ERR_DIMS: return "SV_ERR_DIMS: a dimension is outside the supported limits";
        case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace smaller than sv_workspace_bytes(dims)";
        case SV_ERR_ALIGN: return "SV_ERR_ALIGN: a pointer is not aligned as required";
        case SV_ERR_DEVICE: return "SV_ERR_DEVICE: a HIP kernel launch failed";
    }
    return "unknown sv_status";
}

size_t sv_tiled_w_bytes(int32_t V, int32_t d) {
    return w_shape_ok(V, d) ? sv::tiled_w_bytes(V, d) : 0;
}

sv_status sv_tile_w(const uint16_t* W, int32_t V, int32_t d, uint16_t* W_tiled, size_t tiled_bytes,
                    void* hip_stream) {
    if (!w_shape_ok(V, d)) return SV_ERR_DIMS;
    if (!W || !W_tiled) return SV_ERR_NULL;
    if (!aligned(W, 16) || !aligned(W_tiled, 16)) return SV_ERR_ALIGN;
    if (tiled_bytes < sv::tiled_w_bytes(V, d)) return SV_ERR_WORKSPACE;
    return sv::launch_tile_rows(W, V, d, W_tiled, static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? SV_OK
               : SV_ERR_DEVICE;
}

size_t sv_workspace_bytes(sv_dims dims) {
    if (!dims_ok(dims)) return 0;
    return sv::make_layout(dims.B, dims.gamma, dims.d, dims.V).total;
}

sv_status sv_lmhead(const uint16_t* hidden, const uint16_t* W_lmhead, sv_dims dims, void* workspace,
                    size_t workspace_bytes, void* hip_stream) {
    const sv_status st = check_stage1(hidden, W_lmhead, dims, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    return stage1(hidden, W_lmhead, dims, workspace, static_cast<hipStream_t>(hip_stream));
}

sv_status sv_lmhead_ex(const uint16_t* hidden, const uint16_t* W_lmhead, sv_dims dims, int32_t flags,
                       void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (flags & ~(SV_LMHEAD_LOGITS | SV_LMHEAD_ARGMAX)) return SV_ERR_DIMS;
    const sv_status st = check_stage1(hidden, W_lmhead, dims, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    return stage1(hidden, W_lmhead, dims, workspace, static_cast<hipStream_t>(hip_stream),
                  (flags & SV_LMHEAD_LOGITS) != 0, (flags & SV_LMHEAD_ARGMAX) != 0);
}

sv_status sv_accept_and_draw(const int32_t* draft_tokens, const float* q, const float* uniforms,
                             sv_dims dims, int32_t* out_tokens, int32_t* n_accepted, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
    const sv_status st = check_stage2(draft_tokens, q, uniforms, dims, out_tokens, n_accepted,
                                      workspace, workspace_bytes);
    if (st != SV_OK) return st;
    return stage2(draft_tokens, q, nullptr, 0, uniforms, dims, out_tokens, n_accepted, workspace,
                  static_cast<hipStream_t>(hip_stream));
}

sv_status spec_verify(const uint16_t* hidden, const uint16_t* W_lmhead, const int32_t* draft_tokens,
                      const float* q, const float* uniforms, sv_dims dims, int32_t* out_tokens,
                      int32_t* n_accepted, void* workspace, size_t workspace_bytes, void* hip_stream) {
    sv_status st = check_stage1(hidden, W_lmhead, dims, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    st = check_stage2(draft_tokens, q, uniforms, dims, out_tokens, n_accepted, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = stage1(hidden, W_lmhead, dims, workspace, s, /*keep_logits=*/true, /*with_argmax=*/false);
    if (st != SV_OK) return st;
    return stage2(draft_tokens, q, nullptr, 0, uniforms, dims, out_tokens, n_accepted, workspace, s);
}

sv_status spec_verify_static(const uint16_t* hidden, const uint16_t* W_lmhead,
                             const int32_t* draft_tokens, const float* q, const float* uniforms,
                             sv_dims dims, int32_t* out_tokens, int32_t* n_accepted,
                             void* hip_stream) {
    if (!dims_ok(dims)) return SV_ERR_DIMS;
    if (!hidden || !W_lmhead || !draft_tokens || !q || !uniforms || !out_tokens || !n_accepted)
        return SV_ERR_NULL;
    if (sv_workspace_bytes(dims) > kStaticScratchBytes) return SV_ERR_WORKSPACE;
    void* ws = nullptr;
    const sv_status got = scratch_on_current_device(&ws);
    if (got != SV_OK) return got;
    // The same launches as spec_verify; the LM-head kernel zeroes the
    // per-sequence counters the draw kernels use, so nothing in the array
    // needs clearing first.
    return spec_verify(hidden, W_lmhead, draft_tokens, q, uniforms, dims, out_tokens, n_accepted,
                       ws, kStaticScratchBytes, hip_stream);
}

sv_status sv_accept_and_draw_sparse_q(const int32_t* draft_tokens, const int32_t* q_ids,
                                      const float* q_vals, int32_t K, const float* uniforms,
                                      sv_dims dims, int32_t* out_tokens, int32_t* n_accepted,
                                      void* workspace, size_t workspace_bytes, void* hip_stream) {
    const sv_status st = check_stage2_sparse(draft_tokens, q_ids, q_vals, K, uniforms, dims,
                                             out_tokens, n_accepted, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    return stage2(draft_tokens, q_vals, q_ids, K, uniforms, dims, out_tokens, n_accepted,
                  workspace, static_cast<hipStream_t>(hip_stream));
}

sv_status spec_verify_sparse_q(const uint16_t* hidden, const uint16_t* W_lmhead,
                               const int32_t* draft_tokens, const int32_t* q_ids,
                               const float* q_vals, int32_t K, const float* uniforms,
                               sv_dims dims, int32_t* out_tokens, int32_t* n_accepted,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
    sv_status st = check_stage1(hidden, W_lmhead, dims, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    st = check_stage2_sparse(draft_tokens, q_ids, q_vals, K, uniforms, dims, out_tokens,
                             n_accepted, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = stage1(hidden, W_lmhead, dims, workspace, s, /*keep_logits=*/true, /*with_argmax=*/false);
    if (st != SV_OK) return st;
    return stage2(draft_tokens, q_vals, q_ids, K, uniforms, dims, out_tokens, n_accepted,
                  workspace, s);
}

size_t sv_sparse_head_workspace_bytes(sv_head_dims dims) {
    if (!head_dims_ok(dims)) return 0;
    return sv::make_head_layout(dims.N, dims.C, dims.k * dims.M).total;
}

sv_status sv_sparse_head(const uint16_t* h, const uint16_t* W_lmhead, const uint16_t* centroids,
                         const int32_t* members, sv_head_dims dims, int32_t* q_ids, float* q_vals,
                         int32_t* clusters, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
    if (!head_dims_ok(dims)) return SV_ERR_DIMS;
    if (!h || !W_lmhead || !centroids || !members || !q_ids || !q_vals || !workspace)
        return SV_ERR_NULL;
    if (!aligned(h, 16) || !aligned(W_lmhead, 16) || !aligned(centroids, 16) ||
        !aligned(members, 4) || !aligned(q_ids, 4) || !aligned(q_vals, 4) ||
        !aligned(clusters, 4) || !aligned(workspace, 256))
        return SV_ERR_ALIGN;
    if (workspace_bytes < sv_sparse_head_workspace_bytes(dims)) return SV_ERR_WORKSPACE;
    const hipError_t e = sv::launch_sparse_head(h, W_lmhead, centroids, members, dims.N, dims.d,
                                                dims.V, dims.C, dims.M, dims.k, q_ids, q_vals,
                                                clusters, workspace,
                                                static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_accept_greedy(const int32_t* draft_tokens, sv_dims dims, int32_t* out_tokens,
                           int32_t* n_accepted, int32_t* target_tokens, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
    const sv_status st = check_greedy(draft_tokens, dims, out_tokens, n_accepted, target_tokens,
                                      workspace, workspace_bytes);
    if (st != SV_OK) return st;
    return stage2_greedy(draft_tokens, dims, out_tokens, n_accepted, target_tokens, workspace,
                         static_cast<hipStream_t>(hip_stream));
}

sv_status spec_verify_greedy(const uint16_t* hidden, const uint16_t* W_lmhead,
                             const int32_t* draft_tokens, sv_dims dims, int32_t* out_tokens,
                             int32_t* n_accepted, int32_t* target_tokens, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
    sv_status st = check_stage1(hidden, W_lmhead, dims, workspace, workspace_bytes);
    if (st != SV_OK) return st;
    st = check_greedy(draft_tokens, dims, out_tokens, n_accepted, target_tokens, workspace,
                      workspace_bytes);
    if (st != SV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = stage1(hidden, W_lmhead, dims, workspace, s, /*keep_logits=*/false);
    if (st != SV_OK) return st;
    return stage2_greedy(draft_tokens, dims, out_tokens, n_accepted, target_tokens, workspace, s);
}

sv_status sv_tree_shape(const int32_t* parent, int32_t T, int32_t* depth, int32_t* q_rows,
                        int32_t* rounds) {
    sv::TreeTopo tp;
    int r;
    if (!build_topology(parent, T, &tp, &r)) return SV_ERR_DIMS;
    if (depth) *depth = tp.D;
    if (q_rows) *q_rows = tp.P;
    if (rounds) *rounds = r;
    return SV_OK;
}

size_t sv_tree_workspace_bytes(sv_dims dims) {
    if (!tree_dims_ok(dims)) return 0;
    return sv::make_layout(dims.B, dims.gamma, dims.d, dims.V).total;
}

sv_status spec_verify_tree(const uint16_t* hidden, const uint16_t* W_lmhead, const int32_t* parent,
                           const int32_t* tree_tokens, const float* q, const float* uniforms,
                           sv_dims dims, int32_t* out_tokens, int32_t* n_accepted,
                           int32_t* path_nodes, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    if (!tree_dims_ok(dims)) return SV_ERR_DIMS;
    sv::TreeTopo tp;
    int rounds;
    if (!parent) return SV_ERR_NULL;
    if (!build_topology(parent, dims.gamma, &tp, &rounds)) return SV_ERR_DIMS;
    if (!hidden || !W_lmhead || !tree_tokens || !q || !uniforms || !out_tokens || !n_accepted ||
        !workspace)
        return SV_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(W_lmhead, 16) || !aligned(q, 16) ||
        !aligned(tree_tokens, 4) || !aligned(uniforms, 4) || !aligned(out_tokens, 4) ||
        !aligned(n_accepted, 4) || !aligned(path_nodes, 4) || !aligned(workspace, 256))
        return SV_ERR_ALIGN;
    if (workspace_bytes < sv_tree_workspace_bytes(dims)) return SV_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const sv_status st = stage1(hidden, W_lmhead, dims, workspace, s, /*keep_logits=*/true,
                                /*with_argmax=*/false);
    if (st != SV_OK) return st;
    const sv::Layout L = sv::make_layout(dims.B, dims.gamma, dims.d, dims.V);
    const hipError_t e = sv::launch_tree(
        at<float>(workspace, L.logits), at<float>(workspace, L.part_max),
        at<float>(workspace, L.part_sum), lmhead_partials(L.R, dims.V), L.NPs, dims.B, dims.V, tp,
        rounds, tree_tokens, q, uniforms, L.NC, chunk_sums(workspace, L),
        at<float>(workspace, L.row_max),
        at<float>(workspace, L.row_sum), at<char>(workspace, L.tstate),
        at<int32_t>(workspace, L.counters), out_tokens, n_accepted, path_nodes,
        at<int32_t>(workspace, L.status), s);
    return e == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

sv_status sv_debug_views(const void* workspace, sv_dims dims, const float** logits,
                         const float** row_max, const float** row_sumexp, const int32_t** status) {
    // the dims of a chain call, or of a tree call (gamma = T, up to SV_MAX_TREE_NODES)
    if (!dims_ok(dims) && !tree_dims_ok(dims)) return SV_ERR_DIMS;
    if (!workspace) return SV_ERR_NULL;
    const sv::Layout L = sv::make_layout(dims.B, dims.gamma, dims.d, dims.V);
    const char* base = static_cast<const char*>(workspace);
    if (logits) *logits = reinterpret_cast<const float*>(base + L.logits);
    if (row_max) *row_max = reinterpret_cast<const float*>(base + L.row_max);
    if (row_sumexp) *row_sumexp = reinterpret_cast<const float*>(base + L.row_sum);
    if (status) *status = reinterpret_cast<const int32_t*>(base + L.status);
    return SV_OK;
}

}  // extern "C"
