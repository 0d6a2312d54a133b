// libdecodehp C ABI: argument validation, error reporting and dispatch to the kernel
// launchers. Every check here runs on the host before any HIP call, so a rejected call
// never touches the device.
#include "dhp_internal.hpp"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

namespace {

thread_local char g_err[512] = "";

constexpr int MAX_DEVICES = 64;
std::mutex g_dev_mu;
DeviceFacts g_dev[MAX_DEVICES];
int g_dev_state[MAX_DEVICES];  // 0 unknown, 1 ok, -1 unusable

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and pointer checks for one INT4 tensor; `name` goes into the message.
int check_int4(const dhp_int4* w, const char* name) {
    if (!w) return dhp_fail(DHP_ERR_INVALID, "%s: null descriptor", name);
    if (!w->codes || !w->scales || !w->biases)
        return dhp_fail(DHP_ERR_INVALID, "%s: null codes/scales/biases", name);
    if (w->rows <= 0 || w->cols <= 0)
        return dhp_fail(DHP_ERR_INVALID, "%s: non-positive shape %d x %d", name, w->rows, w->cols);
    if (w->group != 64) return dhp_fail(DHP_ERR_UNSUPPORTED, "%s: group %d (only 64)", name, w->group);
    if (w->cols % 64) return dhp_fail(DHP_ERR_UNSUPPORTED, "%s: cols %d not a multiple of 64", name, w->cols);
    if (!aligned(w->codes, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "%s: codes not 16-byte aligned", name);
    if (!aligned(w->scales, 2) || !aligned(w->biases, 2))
        return dhp_fail(DHP_ERR_MISALIGNED, "%s: scales/biases not 2-byte aligned", name);
    return DHP_OK;
}

int check_experts(const dhp_int4_experts* e, const char* name) {
    if (!e) return dhp_fail(DHP_ERR_INVALID, "%s: null descriptor", name);
    int rc = check_int4(&e->first, name);
    if (rc) return rc;
    if (e->count <= 0) return dhp_fail(DHP_ERR_INVALID, "%s: count %d", name, e->count);
    if (e->codes_stride < 0 || e->scales_stride < 0)
        return dhp_fail(DHP_ERR_INVALID, "%s: negative stride", name);
    if (e->codes_stride % 16) return dhp_fail(DHP_ERR_MISALIGNED, "%s: codes stride %% 16", name);
    if (e->scales_stride % 2) return dhp_fail(DHP_ERR_MISALIGNED, "%s: scales stride %% 2", name);
    return DHP_OK;
}

}  // namespace

int dhp_fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool dhp_current_device(DeviceFacts* out) {
    int dev = -1;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        dhp_fail(DHP_ERR_NO_DEVICE, "no HIP device");
        return false;
    }
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        (void)hipGetLastError();
        dhp_fail(DHP_ERR_NO_DEVICE, "no current HIP device");
        return false;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
            (void)hipGetLastError();
            g_dev_state[dev] = -1;
        } else if (strncmp(p.gcnArchName, "gfx950", 6) != 0) {
            g_dev_state[dev] = -1;
        } else {
            g_dev[dev].device = dev;
            g_dev[dev].cus = p.multiProcessorCount;
            g_dev_state[dev] = 1;
        }
    }
    if (g_dev_state[dev] != 1) {
        dhp_fail(DHP_ERR_NO_DEVICE, "device %d is not a gfx950 GPU", dev);
        return false;
    }
    *out = g_dev[dev];
    return true;
}

size_t dhp_gemv_argmax_ws(int32_t n_rows, int32_t m);
size_t dhp_moe_ws(int32_t n_experts, int32_t top_k, int32_t inter);
size_t dhp_hc_ws(int32_t C, int32_t R);

extern "C" {

const char* decodehp_last_error(void) { return g_err; }

int32_t decodehp_version(void) { return (0 << 16) | 4; }

size_t decodehp_workspace_bytes(int32_t op, int32_t a, int32_t b, int32_t c) {
    switch (op) {
        case DHP_OP_GEMV_ARGMAX: return (a > 0 && b > 0) ? dhp_gemv_argmax_ws(a, b) : 0;
        case DHP_OP_MOE_DECODE: return (a > 0 && b > 0 && c > 0) ? dhp_moe_ws(a, b, c) : 0;
        case DHP_OP_HC_READ: return (a > 0 && b > 0) ? dhp_hc_ws(a, b) : 0;
        default: return 0;
    }
}

}  // extern "C"

namespace {
// Checks shared by the two GEMV entry points.
int check_gemv(const dhp_int4* w, const void* x, int32_t m, const void* y, int32_t y_dtype, const int32_t* argmax,
               const void* ws, size_t ws_bytes) {
    int rc = check_int4(w, "w");
    if (rc) return rc;
    if (!x || !y) return dhp_fail(DHP_ERR_INVALID, "null x or y");
    if (m < 1 || m > DHP_GEMV_MAX_M) return dhp_fail(DHP_ERR_UNSUPPORTED, "m=%d outside 1..%d", m, DHP_GEMV_MAX_M);
    if (y_dtype != DHP_F16 && y_dtype != DHP_F32) return dhp_fail(DHP_ERR_UNSUPPORTED, "y_dtype %d", y_dtype);
    if (w->cols > 16384) return dhp_fail(DHP_ERR_UNSUPPORTED, "K=%d above 16384", w->cols);
    if (!aligned(x, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "x not 16-byte aligned");
    if (!aligned(y, y_dtype == DHP_F32 ? 4 : 2)) return dhp_fail(DHP_ERR_MISALIGNED, "y misaligned");
    if (argmax) {
        if (!aligned(argmax, 4)) return dhp_fail(DHP_ERR_MISALIGNED, "argmax misaligned");
        const size_t need = dhp_gemv_argmax_ws(w->rows, m);
        if (!ws || ws_bytes < need) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
        if (!aligned(ws, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "workspace not 16-byte aligned");
    }
    return DHP_OK;
}
}  // namespace

extern "C" {

int decodehp_dequant_gemv(const dhp_int4* w, const void* x, int32_t m, void* y, int32_t y_dtype,
                          int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    const int rc = check_gemv(w, x, m, y, y_dtype, argmax, ws, ws_bytes);
    if (rc) return rc;
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    if (m == 1)
        return launch_gemv_m1(w, x, y, y_dtype == DHP_F32, argmax, ws, static_cast<hipStream_t>(stream), dev);
    return launch_gemv_rows(w, x, m, y, y_dtype == DHP_F32, argmax, ws, dhp_argmax_part_stride(w->rows, m),
                            static_cast<hipStream_t>(stream), dev.cus);
}

int decodehp_dequant_gemv_mc(const dhp_int4* w, const void* x, int32_t m, void* y, int32_t y_dtype,
                             int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    const int rc = check_gemv(w, x, m, y, y_dtype, argmax, ws, ws_bytes);
    if (rc) return rc;
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    if (dhp_gemv_mfma16_fits(w, m))
        return launch_gemv_mfma16(w, x, m, y, y_dtype == DHP_F32, argmax, ws, dhp_argmax_part_stride(w->rows, m),
                                  static_cast<hipStream_t>(stream), dev.cus);
    return launch_gemm_mfma(w, x, m, y, y_dtype == DHP_F32, argmax, ws, dhp_argmax_part_stride(w->rows, m),
                            static_cast<hipStream_t>(stream));
}

int decodehp_dequant_gemm_batched(const dhp_int4* w, const void* x, int32_t m, void* y, void* stream) {
    g_err[0] = 0;
    int rc = check_int4(w, "w");
    if (rc) return rc;
    if (!x || !y) return dhp_fail(DHP_ERR_INVALID, "null x or y");
    if (m < 1 || m > DHP_GEMM_MAX_M) return dhp_fail(DHP_ERR_UNSUPPORTED, "m=%d outside 1..%d", m, DHP_GEMM_MAX_M);
    if (w->rows % 16) return dhp_fail(DHP_ERR_UNSUPPORTED, "N=%d not a multiple of 16", w->rows);
    if (w->cols > 32768) return dhp_fail(DHP_ERR_UNSUPPORTED, "K=%d above 32768", w->cols);
    if (!aligned(x, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "x not 16-byte aligned");
    if (!aligned(y, 2)) return dhp_fail(DHP_ERR_MISALIGNED, "y misaligned");
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_gemm_mfma(w, x, m, y, 0, nullptr, nullptr, 0, static_cast<hipStream_t>(stream));
}

namespace {
// Checks shared by the MoE entry points: shapes, limits, dtypes, flags and alignment of the
// weights and of x/out/ids/weights (x is 16-byte aligned; rows of x and out then stay aligned
// because hidden is a multiple of 512).
int check_moe(const void* x, const void* router, int32_t router_dtype, const void* shared_gate_row,
              const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
              const dhp_int4* shared_gate, const dhp_int4* shared_up, const dhp_int4* shared_down,
              int32_t top_k, int32_t flags, const void* out, const int32_t* ids, const float* weights) {
    if (!x || !router || !shared_gate_row || !out || !ids || !weights)
        return dhp_fail(DHP_ERR_INVALID, "null x, router, shared_gate_row, out, ids or weights");
    int rc = check_experts(gate, "gate");
    if (!rc) rc = check_experts(up, "up");
    if (!rc) rc = check_experts(down, "down");
    if (!rc) rc = check_int4(shared_gate, "shared_gate");
    if (!rc) rc = check_int4(shared_up, "shared_up");
    if (!rc) rc = check_int4(shared_down, "shared_down");
    if (rc) return rc;
    const int hidden = gate->first.cols, inter = gate->first.rows, E = gate->count;
    if (up->first.rows != inter || up->first.cols != hidden || up->count != E)
        return dhp_fail(DHP_ERR_INVALID, "up experts do not match gate (%d x %d x %d)", E, inter, hidden);
    if (down->first.rows != hidden || down->first.cols != inter || down->count != E)
        return dhp_fail(DHP_ERR_INVALID, "down experts must be %d x [%d x %d]", E, hidden, inter);
    if (shared_gate->rows != inter || shared_gate->cols != hidden || shared_up->rows != inter ||
        shared_up->cols != hidden || shared_down->rows != hidden || shared_down->cols != inter)
        return dhp_fail(DHP_ERR_INVALID, "shared expert shapes must match the routed experts");
    if (hidden % 512 || hidden > 4096)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "hidden=%d (a multiple of 512, at most 4096)", hidden);
    if (inter > 1024) return dhp_fail(DHP_ERR_UNSUPPORTED, "inter=%d above 1024", inter);
    if (E > 1024) return dhp_fail(DHP_ERR_UNSUPPORTED, "n_experts=%d above 1024", E);
    if (top_k < 1 || top_k > DHP_MOE_MAX_TOP_K || top_k > E)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "top_k=%d (1..%d and at most n_experts=%d)", top_k, DHP_MOE_MAX_TOP_K, E);
    if (router_dtype != DHP_BF16 && router_dtype != DHP_F32 && router_dtype != DHP_I8)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "router_dtype %d (bf16, fp32 or int8)", router_dtype);
    if (flags & ~DHP_MOE_FP16_BOUNDARY) return dhp_fail(DHP_ERR_UNSUPPORTED, "flags 0x%x", flags);
    if (!aligned(x, 16) || !aligned(router, router_dtype == DHP_I8 ? 8 : 16) || !aligned(shared_gate_row, 16))
        return dhp_fail(DHP_ERR_MISALIGNED, "x and shared_gate_row must be 16-byte aligned, router rows 16 (int8: 8)");
    if (!aligned(out, 2) || !aligned(ids, 4) || !aligned(weights, 4))
        return dhp_fail(DHP_ERR_MISALIGNED, "out, ids or weights misaligned");
    return DHP_OK;
}
}  // namespace

namespace {
int check_router_scales(const dhp_router* r) {
    if (r->elem_scale && !aligned(r->elem_scale, 16))
        return dhp_fail(DHP_ERR_MISALIGNED, "router elem_scale not 16-byte aligned");
    if (r->expert_scale && !aligned(r->expert_scale, 4))
        return dhp_fail(DHP_ERR_MISALIGNED, "router expert_scale misaligned");
    return DHP_OK;
}

int moe_decode_impl(const void* x, const dhp_router* router, const void* shared_gate_row,
                    const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
                    const dhp_int4* shared_gate, const dhp_int4* shared_up, const dhp_int4* shared_down,
                    int32_t top_k, int32_t flags, void* out, int32_t* ids, float* weights, void* ws,
                    size_t ws_bytes, void* stream) {
    int rc = check_moe(x, router->weights, router->dtype, shared_gate_row, gate, up, down, shared_gate, shared_up,
                       shared_down, top_k, flags, out, ids, weights);
    if (!rc) rc = check_router_scales(router);
    if (rc) return rc;
    const size_t need = dhp_moe_ws(gate->count, top_k, gate->first.rows);
    if (!ws || ws_bytes < need) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "workspace not 16-byte aligned");
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_moe(x, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k,
                      (flags & DHP_MOE_FP16_BOUNDARY) != 0, out, ids, weights, ws, static_cast<hipStream_t>(stream));
}

int moe_prefill_impl(const void* x, int32_t m, const dhp_router* router, const void* shared_gate_row,
                     const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
                     const dhp_int4* shared_gate, const dhp_int4* shared_up, const dhp_int4* shared_down,
                     int32_t top_k, int32_t flags, void* out, int32_t* ids, float* weights, void* ws,
                     size_t ws_bytes, void* stream) {
    if (m < 1 || m > DHP_MOE_PREFILL_MAX_M)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "m=%d (1..%d)", m, DHP_MOE_PREFILL_MAX_M);
    int rc = check_moe(x, router->weights, router->dtype, shared_gate_row, gate, up, down, shared_gate, shared_up,
                       shared_down, top_k, flags, out, ids, weights);
    if (!rc) rc = check_router_scales(router);
    if (rc) return rc;
    const size_t need = dhp_moe_prefill_ws(m, gate->count, top_k, gate->first.rows, gate->first.cols);
    if (!ws || ws_bytes < need) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "workspace not 16-byte aligned");
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_moe_prefill(x, m, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down,
                              top_k, (flags & DHP_MOE_FP16_BOUNDARY) != 0, out, ids, weights, ws,
                              static_cast<hipStream_t>(stream));
}
}  // namespace

int decodehp_moe_decode(const void* x, const void* router, int32_t router_dtype,
                        const void* shared_gate_row, const dhp_int4_experts* gate,
                        const dhp_int4_experts* up, const dhp_int4_experts* down,
                        const dhp_int4* shared_gate, const dhp_int4* shared_up,
                        const dhp_int4* shared_down, int32_t top_k, int32_t flags, void* out,
                        int32_t* ids, float* weights, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    const dhp_router r{router, router_dtype, nullptr, nullptr};
    return moe_decode_impl(x, &r, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k, flags,
                           out, ids, weights, ws, ws_bytes, stream);
}

int decodehp_moe_decode_ex(const void* x, const dhp_router* router, const void* shared_gate_row,
                           const dhp_int4_experts* gate, const dhp_int4_experts* up,
                           const dhp_int4_experts* down, const dhp_int4* shared_gate,
                           const dhp_int4* shared_up, const dhp_int4* shared_down, int32_t top_k,
                           int32_t flags, void* out, int32_t* ids, float* weights, void* ws,
                           size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!router) return dhp_fail(DHP_ERR_INVALID, "null router");
    return moe_decode_impl(x, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k,
                           flags, out, ids, weights, ws, ws_bytes, stream);
}

}  // extern "C"

// Scratch of decodehp_moe_decode_noalloc: one array per GPU, allocated with the code object when
// the library loads on that device and held until the process ends. Host code never takes the
// array's name as a device address: hipGetSymbolAddress gives each device's own copy, once per
// device (with that device current, on the entry point's first call there), and that address is
// what the launch receives.
namespace {
__device__ __align__(256) unsigned char scratch[DHP_NOALLOC_SCRATCH_BYTES];
void* g_scratch_addr[MAX_DEVICES];

void* scratch_address(int dev) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            dhp_fail(DHP_ERR_LAUNCH, "scratch address on device %d: %s", dev, hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_addr[dev] = p;
    }
    return g_scratch_addr[dev];
}
}  // namespace

extern "C" {

int decodehp_moe_decode_noalloc(const void* x, const void* router, int32_t router_dtype,
                                const void* shared_gate_row, const dhp_int4_experts* gate,
                                const dhp_int4_experts* up, const dhp_int4_experts* down,
                                const dhp_int4* shared_gate, const dhp_int4* shared_up,
                                const dhp_int4* shared_down, int32_t top_k, int32_t flags, void* out,
                                int32_t* ids, float* weights, void* stream) {
    g_err[0] = 0;
    int rc = check_moe(x, router, router_dtype, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down,
                       top_k, flags, out, ids, weights);
    if (rc) return rc;
    const size_t need = dhp_moe_ws(gate->count, top_k, gate->first.rows);
    if (need > DHP_NOALLOC_SCRATCH_BYTES)
        return dhp_fail(DHP_ERR_WORKSPACE,
                        "the layer needs %zu bytes of scratch (n_experts %d, top_k %d, inter %d); the library's "
                        "own scratch holds %d: call decodehp_moe_decode with a workspace",
                        need, gate->count, top_k, gate->first.rows, DHP_NOALLOC_SCRATCH_BYTES);
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    void* ws = scratch_address(dev.device);
    if (!ws) return DHP_ERR_LAUNCH;
    const dhp_router r{router, router_dtype, nullptr, nullptr};
    // the router logits, the gate logit and the activations in the scratch are each written before
    // they are read within the call, so nothing there needs clearing between calls
    return launch_moe(x, &r, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k,
                      (flags & DHP_MOE_FP16_BOUNDARY) != 0, out, ids, weights, ws, static_cast<hipStream_t>(stream));
}

size_t decodehp_moe_prefill_workspace_bytes(int32_t m, int32_t n_experts, int32_t top_k, int32_t inter,
                                            int32_t hidden) {
    if (m < 1 || m > DHP_MOE_PREFILL_MAX_M || n_experts < 1 || n_experts > 1024 || top_k < 1 ||
        top_k > DHP_MOE_MAX_TOP_K || inter < 1 || inter > 1024 || hidden < 1 || hidden > 4096)
        return 0;
    return dhp_moe_prefill_ws(m, n_experts, top_k, inter, hidden);
}

int decodehp_moe_prefill(const void* x, int32_t m, const void* router, int32_t router_dtype,
                         const void* shared_gate_row, const dhp_int4_experts* gate,
                         const dhp_int4_experts* up, const dhp_int4_experts* down,
                         const dhp_int4* shared_gate, const dhp_int4* shared_up,
                         const dhp_int4* shared_down, int32_t top_k, int32_t flags, void* out,
                         int32_t* ids, float* weights, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    const dhp_router r{router, router_dtype, nullptr, nullptr};
    return moe_prefill_impl(x, m, &r, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k,
                            flags, out, ids, weights, ws, ws_bytes, stream);
}

int decodehp_moe_prefill_ex(const void* x, int32_t m, const dhp_router* router, const void* shared_gate_row,
                            const dhp_int4_experts* gate, const dhp_int4_experts* up,
                            const dhp_int4_experts* down, const dhp_int4* shared_gate,
                            const dhp_int4* shared_up, const dhp_int4* shared_down, int32_t top_k,
                            int32_t flags, void* out, int32_t* ids, float* weights, void* ws,
                            size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!router) return dhp_fail(DHP_ERR_INVALID, "null router");
    return moe_prefill_impl(x, m, router, shared_gate_row, gate, up, down, shared_gate, shared_up, shared_down, top_k,
                            flags, out, ids, weights, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {
// Checks shared by the single-token and batched hyper-connection reads.
int check_hc_read(const void* raw, const void* hc_norm, int32_t C, int32_t H, float eps, const dhp_int4* down,
                  const dhp_int4* up, const dhp_int4* inject, const void* mixed, const float* inject_w) {
    if (!raw || !hc_norm || !mixed) return dhp_fail(DHP_ERR_INVALID, "null raw, hc_norm or mixed");
    if (C <= 0 || H <= 0) return dhp_fail(DHP_ERR_INVALID, "C=%d H=%d", C, H);
    if (C > DHP_HC_MAX_C || (C & (C - 1)))
        return dhp_fail(DHP_ERR_UNSUPPORTED, "C=%d (a power of two up to %d)", C, DHP_HC_MAX_C);
    if (H % 64) return dhp_fail(DHP_ERR_UNSUPPORTED, "H=%d not a multiple of 64", H);
    const long wide = (long)C * H;
    if (wide % 2048 || wide > 32768)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "C*H=%ld (a multiple of 2048, at most 32768)", wide);
    if (!(eps >= 0.0f) || eps > 1.0f) return dhp_fail(DHP_ERR_INVALID, "eps %g", (double)eps);
    int rc = check_int4(down, "down");
    if (rc) return rc;
    rc = check_int4(up, "up");
    if (rc) return rc;
    const int R = down->rows;
    if (down->cols != wide) return dhp_fail(DHP_ERR_INVALID, "down is %d x %d, expected R x %ld", down->rows, down->cols, wide);
    if (R % 64 || R > 1024) return dhp_fail(DHP_ERR_UNSUPPORTED, "R=%d (a multiple of 64, at most 1024)", R);
    if (up->rows != wide || up->cols != R)
        return dhp_fail(DHP_ERR_INVALID, "up is %d x %d, expected %ld x %d", up->rows, up->cols, wide, R);
    if (inject) {
        rc = check_int4(inject, "inject");
        if (rc) return rc;
        if (inject->rows != C || inject->cols != wide)
            return dhp_fail(DHP_ERR_INVALID, "inject is %d x %d, expected %d x %ld", inject->rows, inject->cols, C, wide);
        if (!inject_w) return dhp_fail(DHP_ERR_INVALID, "inject given but inject_w is null");
        if (!aligned(inject_w, 4)) return dhp_fail(DHP_ERR_MISALIGNED, "inject_w misaligned");
    } else if (inject_w) {
        return dhp_fail(DHP_ERR_INVALID, "inject_w given without an inject projection");
    }
    if (!aligned(raw, 16) || !aligned(hc_norm, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "raw/hc_norm not 16-byte aligned");
    if (!aligned(mixed, 2)) return dhp_fail(DHP_ERR_MISALIGNED, "mixed misaligned");
    return DHP_OK;
}

int check_hc_inject(const void* wide, const void* out, const float* inject_w, int32_t C, int32_t H) {
    if (!wide || !out || !inject_w) return dhp_fail(DHP_ERR_INVALID, "null wide, out or inject_w");
    if (C <= 0 || H <= 0) return dhp_fail(DHP_ERR_INVALID, "C=%d H=%d", C, H);
    if (C > DHP_HC_MAX_C) return dhp_fail(DHP_ERR_UNSUPPORTED, "C=%d above %d", C, DHP_HC_MAX_C);
    if (H % 8) return dhp_fail(DHP_ERR_UNSUPPORTED, "H=%d not a multiple of 8", H);
    if (!aligned(wide, 16) || !aligned(out, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "wide/out not 16-byte aligned");
    if (!aligned(inject_w, 4)) return dhp_fail(DHP_ERR_MISALIGNED, "inject_w misaligned");
    return DHP_OK;
}
}  // namespace

extern "C" {

int decodehp_hc_read(const void* raw, const void* hc_norm, int32_t C, int32_t H, float eps,
                     const dhp_int4* down, const dhp_int4* up, const dhp_int4* inject,
                     void* mixed, float* inject_w, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    const int rc = check_hc_read(raw, hc_norm, C, H, eps, down, up, inject, mixed, inject_w);
    if (rc) return rc;
    const size_t need = dhp_hc_ws(C, down->rows);
    if (!ws || ws_bytes < need) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "workspace not 16-byte aligned");
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_hc_read(raw, hc_norm, C, H, eps, down, up, inject, mixed, inject_w, ws,
                          static_cast<hipStream_t>(stream));
}

int decodehp_hc_inject(void* wide, const void* out, const float* inject_w, int32_t C, int32_t H,
                       void* stream) {
    g_err[0] = 0;
    const int rc = check_hc_inject(wide, out, inject_w, C, H);
    if (rc) return rc;
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_hc_inject(wide, out, inject_w, C, H, static_cast<hipStream_t>(stream));
}

int decodehp_hc_inject_read(const void* prev, const void* out, const float* inject_w, void* hidden,
                            const void* hc_norm, int32_t C, int32_t H, float eps, const dhp_int4* down,
                            const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w_next,
                            void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_hc_inject(prev, out, inject_w, C, H);
    if (!rc) rc = check_hc_inject(hidden, out, inject_w, C, H);
    if (!rc) rc = check_hc_read(hidden, hc_norm, C, H, eps, down, up, inject, mixed, inject_w_next);
    if (rc) return rc;
    const uintptr_t wide = (uintptr_t)C * H * 2;
    auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
        const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
        return pa < pb + nb && pb < pa + na;
    };
    if (overlap(hidden, wide, prev, wide) || overlap(hidden, wide, out, (uintptr_t)H * 2))
        return dhp_fail(DHP_ERR_INVALID, "hidden overlaps prev or out");
    if (inject_w_next && overlap(inject_w_next, (uintptr_t)C * 4, inject_w, (uintptr_t)C * 4))
        return dhp_fail(DHP_ERR_INVALID, "inject_w_next overlaps inject_w");
    const size_t need = dhp_hc_ws(C, down->rows);
    if (!ws || ws_bytes < need) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "workspace not 16-byte aligned");
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_hc_inject_read(prev, out, inject_w, hidden, hc_norm, C, H, eps, down, up, inject, mixed,
                                 inject_w_next, ws, static_cast<hipStream_t>(stream));
}

size_t decodehp_hc_read_batched_workspace_bytes(int32_t m, int32_t C, int32_t H, int32_t R) {
    if (m < 1 || m > DHP_GEMM_MAX_M || C < 1 || C > DHP_HC_MAX_C || H < 1 || R < 1 || R > 1024) return 0;
    return dhp_hc_read_batched_ws(m, C, H, R);
}

int decodehp_hc_read_batched(const void* raw, int32_t m, const void* hc_norm, int32_t C, int32_t H, float eps,
                             const dhp_int4* down, const dhp_int4* up, const dhp_int4* inject, void* mixed,
                             float* inject_w, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (m < 1 || m > DHP_GEMM_MAX_M) return dhp_fail(DHP_ERR_UNSUPPORTED, "m=%d (1..%d)", m, DHP_GEMM_MAX_M);
    const int rc = check_hc_read(raw, hc_norm, C, H, eps, down, up, inject, mixed, inject_w);
    if (rc) return rc;
    if (!aligned(mixed, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "mixed not 16-byte aligned");
    const size_t need = dhp_hc_read_batched_ws(m, C, H, down->rows);
    if (!ws || ws_bytes < need) return dhp_fail(DHP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 16)) return dhp_fail(DHP_ERR_MISALIGNED, "workspace not 16-byte aligned");
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_hc_read_batched(raw, m, hc_norm, C, H, eps, down, up, inject, mixed, inject_w, ws,
                                  static_cast<hipStream_t>(stream));
}

int decodehp_hc_inject_batched(void* wide, int32_t m, const void* out, const float* inject_w, int32_t C,
                               int32_t H, void* stream) {
    g_err[0] = 0;
    if (m < 1 || m > DHP_GEMM_MAX_M) return dhp_fail(DHP_ERR_UNSUPPORTED, "m=%d (1..%d)", m, DHP_GEMM_MAX_M);
    const int rc = check_hc_inject(wide, out, inject_w, C, H);
    if (rc) return rc;
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    return launch_hc_inject_batched(wide, m, out, inject_w, C, H, static_cast<hipStream_t>(stream));
}

}  // extern "C"

