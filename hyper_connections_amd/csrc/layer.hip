// Whole decoder layers for one token, run as a launch sequence on one stream or replayed as one
// captured HIP graph.
//
// "src/families/qwen4/mod.rs" (turbospark-runtime 0.3.0), module doc, "The decoder layer, as
// pseudocode": the token's hidden vector is replicated over the C streams at entry; each layer
// runs the attn_hc read, the attention sublayer, the inject, the mlp_hc read, the MoE and the
// inject; the hyper_connection_mixer (a read with no inject projection) closes the stack. The
// inject adds the sublayer output to the un-normalized residual ("THE INJECTION TRAP").
// The attention sublayer is not built here: an INT4 [H x H] map stands in for it.
//
// Every step is the library's own entry point (so each keeps its checks), called in order on the
// stream; the only kernel of this file replicates the token at entry. Each inject is fused into
// the read that follows it (decodehp_hc_inject_read), so the inject costs no launch of its own;
// the fused read writes the injected residual to a second buffer, and the two buffers alternate.
// The graph form is the counterpart of the pages' one command buffer per token
// ("src/real_forward.rs", module doc): a decode layer is 8 dependent launches, and replaying them
// as one graph removes the host's per-launch work from the token's critical path.
#include "dhp_internal.hpp"

#include <algorithm>
#include <new>

namespace {

__global__ __launch_bounds__(256) void k_replicate(const uint4* __restrict__ x, uint4* __restrict__ hidden,
                                                   int n16, int total16) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < total16) hidden[i] = x[i % n16];
}

size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }

struct LayerWs {
    size_t scratch, mixed, out, iw, iw2, resid, ids, wts, total;
};

bool block_ok(const dhp_hc_block* b, bool inject) {
    return b && b->hc_norm && b->down && b->up && ((b->inject != nullptr) == inject);
}

// Workspace layout: one scratch region shared by every step (they run in order on one stream),
// then the step outputs the next step reads: mixed fp16 [H], the sublayer/MoE output fp16 [H],
// two sets of inject weights fp32 [C] (a fused inject-read consumes one and writes the other),
// the second residual buffer fp16 [C*H], and the MoE ids and weights (not returned).
bool layer_ws(int C, int H, const dhp_decode_layer* layers, int n, const dhp_hc_block* mixer, LayerWs* w) {
    if (C <= 0 || H <= 0 || n < 0 || (n > 0 && !layers) || !block_ok(mixer, false)) return false;
    size_t scratch = decodehp_workspace_bytes(DHP_OP_HC_READ, C, mixer->down->rows, 0);
    for (int i = 0; i < n; ++i) {
        const dhp_decode_layer& L = layers[i];
        if (!block_ok(&L.attn_hc, true) || !block_ok(&L.mlp_hc, true) || !L.sublayer || !L.gate) return false;
        scratch = std::max(scratch, decodehp_workspace_bytes(DHP_OP_HC_READ, C, L.attn_hc.down->rows, 0));
        scratch = std::max(scratch, decodehp_workspace_bytes(DHP_OP_HC_READ, C, L.mlp_hc.down->rows, 0));
        scratch = std::max(scratch, decodehp_workspace_bytes(DHP_OP_MOE_DECODE, L.gate->count, L.top_k,
                                                             L.gate->first.rows));
    }
    w->scratch = 0;
    w->mixed = a256(scratch);
    w->out = w->mixed + a256((size_t)H * 2);
    w->iw = w->out + a256((size_t)H * 2);
    w->iw2 = w->iw + a256((size_t)C * 4);
    w->resid = w->iw2 + a256((size_t)C * 4);
    w->ids = w->resid + a256((size_t)C * H * 2);
    w->wts = w->ids + a256((size_t)DHP_MOE_MAX_TOP_K * 4);
    w->total = w->wts + a256((size_t)DHP_MOE_MAX_TOP_K * 4);
    return true;
}

int run_layers(const void* x, int C, int H, float eps, const dhp_decode_layer* layers, int n,
               const dhp_hc_block* mixer, void* hidden, void* mixed_out, void* ws, size_t ws_bytes,
               hipStream_t s) {
    LayerWs w;
    if (!layer_ws(C, H, layers, n, mixer, &w))
        return dhp_fail(DHP_ERR_INVALID, "null or inconsistent layer descriptors (C=%d H=%d n=%d)", C, H, n);
    if (!x || !hidden || !mixed_out) return dhp_fail(DHP_ERR_INVALID, "null x, hidden or mixed_out");
    if (H % 64) return dhp_fail(DHP_ERR_UNSUPPORTED, "H=%d not a multiple of 64", H);
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(hidden) |
         reinterpret_cast<uintptr_t>(ws)) % 16)
        return dhp_fail(DHP_ERR_MISALIGNED, "x, hidden and ws must be 16-byte aligned");
    if (!ws || ws_bytes < w.total) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
    char* base = static_cast<char*>(ws);
    void* scratch = base + w.scratch;
    const size_t scratch_bytes = w.mixed - w.scratch;
    void* mixed = base + w.mixed;
    void* out = base + w.out;
    float* iw_buf[2] = {reinterpret_cast<float*>(base + w.iw), reinterpret_cast<float*>(base + w.iw2)};
    void* resid[2] = {hidden, base + w.resid};
    int32_t* ids = reinterpret_cast<int32_t*>(base + w.ids);
    float* wts = reinterpret_cast<float*>(base + w.wts);

    const int n16 = H / 8, total16 = C * n16;
    hipLaunchKernelGGL(k_replicate, dim3((total16 + 255) / 256), dim3(256), 0, s, static_cast<const uint4*>(x),
                       static_cast<uint4*>(hidden), n16, total16);
    const hipError_t le = hipGetLastError();
    int rc = (le == hipSuccess) ? DHP_OK : dhp_fail(DHP_ERR_LAUNCH, "replicate launch: %s", hipGetErrorString(le));
    // cur: the buffer holding the residual; gi: the inject weights the pending inject uses. A read
    // with an inject pending is the fused inject-read: it forms resid[cur ^ 1] and writes the new
    // gates to iw_buf[gi ^ 1]. 2 * n injects in all, so the residual ends in resid[0] = hidden.
    int cur = 0, gi = 0;
    bool pending = false;
    auto read = [&](const dhp_hc_block* b, void* mixed_to, bool with_inject) {
        float* next_iw = with_inject ? iw_buf[pending ? gi ^ 1 : gi] : nullptr;
        int r;
        if (pending) {
            r = decodehp_hc_inject_read(resid[cur], out, iw_buf[gi], resid[cur ^ 1], b->hc_norm, C, H, eps, b->down,
                                        b->up, b->inject, mixed_to, next_iw, scratch, scratch_bytes, s);
            cur ^= 1;
            gi ^= 1;
        } else {
            r = decodehp_hc_read(resid[cur], b->hc_norm, C, H, eps, b->down, b->up, b->inject, mixed_to, next_iw,
                                 scratch, scratch_bytes, s);
        }
        pending = false;
        return r;
    };
    for (int i = 0; i < n && !rc; ++i) {
        const dhp_decode_layer& L = layers[i];
        rc = read(&L.attn_hc, mixed, true);
        if (!rc) rc = decodehp_dequant_gemv(L.sublayer, mixed, 1, out, DHP_F16, nullptr, nullptr, 0, s);
        pending = true;
        if (!rc) rc = read(&L.mlp_hc, mixed, true);
        if (!rc)
            rc = decodehp_moe_decode(mixed, L.router, L.router_dtype, L.shared_gate_row, L.gate, L.up, L.down,
                                     L.shared_gate, L.shared_up, L.shared_down, L.top_k, L.moe_flags, out, ids, wts,
                                     scratch, scratch_bytes, s);
        pending = true;
    }
    if (!rc) rc = read(mixer, mixed_out, false);
    return rc;
}

}  // namespace

struct dhp_graph {
    hipGraphExec_t exec;
};

extern "C" {

size_t decodehp_decode_layers_workspace_bytes(int32_t C, int32_t H, const dhp_decode_layer* layers,
                                              int32_t n_layers, const dhp_hc_block* mixer) {
    LayerWs w;
    return layer_ws(C, H, layers, n_layers, mixer, &w) ? w.total : 0;
}

int decodehp_decode_layers(const void* x, int32_t C, int32_t H, float eps, const dhp_decode_layer* layers,
                           int32_t n_layers, const dhp_hc_block* mixer, void* hidden, void* mixed_out,
                           void* ws, size_t ws_bytes, void* stream) {
    return run_layers(x, C, H, eps, layers, n_layers, mixer, hidden, mixed_out, ws, ws_bytes,
                      static_cast<hipStream_t>(stream));
}

int decodehp_graph_capture_decode_layers(const void* x, int32_t C, int32_t H, float eps,
                                         const dhp_decode_layer* layers, int32_t n_layers,
                                         const dhp_hc_block* mixer, void* hidden, void* mixed_out,
                                         void* ws, size_t ws_bytes, dhp_graph** graph) {
    if (!graph) return dhp_fail(DHP_ERR_INVALID, "null graph handle");
    *graph = nullptr;
    // the inputs may have been written by asynchronous work on any stream: wait for all of it
    if (hipDeviceSynchronize() != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "device synchronization failed");
    hipStream_t cs;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess)
        return dhp_fail(DHP_ERR_LAUNCH, "stream creation failed");
    // one eager pass first: every step configures its kernels (LDS limits, occupancy) outside
    // the capture, and argument errors surface before anything is recorded
    int rc = run_layers(x, C, H, eps, layers, n_layers, mixer, hidden, mixed_out, ws, ws_bytes, cs);
    if (!rc && hipStreamSynchronize(cs) != hipSuccess) rc = dhp_fail(DHP_ERR_LAUNCH, "eager pass failed");
    hipGraph_t g = nullptr;
    if (!rc) {
        if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
            rc = dhp_fail(DHP_ERR_LAUNCH, "capture could not start");
        } else {
            rc = run_layers(x, C, H, eps, layers, n_layers, mixer, hidden, mixed_out, ws, ws_bytes, cs);
            const hipError_t e = hipStreamEndCapture(cs, &g);       // always ends the capture
            if (!rc && (e != hipSuccess || !g)) rc = dhp_fail(DHP_ERR_LAUNCH, "capture failed: %s", hipGetErrorString(e));
        }
    }
    hipGraphExec_t exec = nullptr;
    if (!rc && hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess)
        rc = dhp_fail(DHP_ERR_LAUNCH, "graph instantiation failed");
    if (g) hipGraphDestroy(g);
    hipStreamDestroy(cs);
    if (rc) return rc;
    dhp_graph* h = new (std::nothrow) dhp_graph{exec};
    if (!h) {
        hipGraphExecDestroy(exec);
        return dhp_fail(DHP_ERR_LAUNCH, "out of host memory");
    }
    *graph = h;
    return DHP_OK;
}

int decodehp_graph_launch(const dhp_graph* graph, void* stream) {
    if (!graph) return dhp_fail(DHP_ERR_INVALID, "null graph");
    const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "graph launch: %s", hipGetErrorString(e));
    return DHP_OK;
}

void decodehp_graph_destroy(dhp_graph* graph) {
    if (!graph) return;
    hipGraphExecDestroy(graph->exec);
    delete graph;
}

}  // extern "C"
