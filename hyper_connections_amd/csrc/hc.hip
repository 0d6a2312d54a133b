// Hyper-connection read (grouped RMS norm, low-rank mix, inject gate) and inject add.
//
// "src/families/qwen4/mod.rs" (turbospark-runtime 0.3.0), section Hyper-connections, and
// "src/families/qwen4/hc.rs", encode_hyper_connection. The pages run one dispatch per
// step (norm, down GEMV, scale by 1/C, SiLU, up GEMV, sigmoid, mix, inject GEMV, scale,
// sigmoid, scale by 2). Here the read is two kernels:
//
//  k_hc_down : one block per output row of the down projection (R rows) and of the inject
//              projection (C rows), C*H/32 lanes wide (lane t owns input positions 32t..32t+31).
//              Each lane dots its slice of the weight row with raw * hc_norm and sums its squares;
//              per stream, the dot is scaled by the stream's inverse RMS afterwards, so the norm is
//              off the dot's path (every block recomputes the C RMS values from the 20 KB residual,
//              an L2 hit). The epilogue applies the 1/C, then SiLU (down rows) or 2*sigmoid
//              (inject rows). A variant forms the residual first from the previous sublayer's
//              inject (raw + out * inject_w, rounded to fp16) and stores it.
//  k_hc_up   : 16 lanes per output position h: 16/C lanes per stream row c*H+h walk that row's
//              R/32 code chunks against the low-rank vector staged in LDS, the row sums go
//              through the sigmoid, multiply the recomputed normed value, and the C products
//              are averaged.
//
// The normalized stream is never written to memory; only lo [R] and the C inverse RMS
// values pass between the two kernels through the workspace.
#include "dhp_internal.hpp"

namespace {

constexpr int HC_MAX_THREADS = 1024;
constexpr int LO_PITCH = 36;           // floats per staged 32-float chunk of the low-rank vector
constexpr int UP_THREADS = 64;         // k_hc_up block: four outputs h

// One block per projection row (down rows first, then inject rows), C*H/32 lanes: lane t owns
// positions 32t .. 32t+31 of the residual, all in stream c = t / (H/32). With the norm weight
// applied but not yet the stream's inverse RMS, each lane forms
//     P_t = s * (q . v) + b * sum(v),   v = raw * gamma   (its share of the row's dot with raw*gamma)
//     S_t = sum(raw^2)                                     (its share of the stream's sum of squares)
// The inverse RMS is constant within a stream, so the row's dot with the normed residual is
//     sum_c ir_c * P_c,   P_c, S_c = the stream's sums of P_t, S_t,   ir_c = 1 / sqrt(S_c / H + eps).
// The dot therefore does not wait for the norm: every load is issued up front and the block meets
// once (sums within 16-lane groups by DPP, then one LDS exchange), then the epilogue applies the
// 1/C and SiLU (down rows) or 2*sigmoid (inject rows).
// INJ: the previous sublayer's inject is fused in front. Each lane first forms its residual values
// as fp16(raw_prev + out[h] * iw[c]) with inject_pair, as k_hc_inject does, so the values are the
// same bits the separate inject would store, and block 0 stores them to `hidden` (which must not
// overlap raw_prev: the other blocks are still reading it).
template <bool INJ>
__global__ __launch_bounds__(HC_MAX_THREADS) void k_hc_down(
    const _Float16* __restrict__ raw, const uint16_t* __restrict__ gamma, int C, int H, float eps,
    const u32x4* __restrict__ dcodes, const uint16_t* __restrict__ dscales,
    const uint16_t* __restrict__ dbiases, int R, const u32x4* __restrict__ icodes,
    const uint16_t* __restrict__ iscales, const uint16_t* __restrict__ ibiases,
    const _Float16* __restrict__ inj_out, const float* __restrict__ inj_w, _Float16* __restrict__ hidden,
    float* __restrict__ lo_out, float* __restrict__ inv_rms_out, float* __restrict__ inject_w) {
    __shared__ float2 part[HC_MAX_THREADS];

    const int t = threadIdx.x;            // chunk index, input positions 32t .. 32t+31
    const int G = (C * H) >> 6;
    const int per = H >> 5;               // chunks (lanes) per stream
    const int c = t / per;                // this lane's stream
    const int row = blockIdx.x;
    const bool is_inject = row >= R;
    const int r = is_inject ? row - R : row;

    // every load up front: the weight slice, the residual (and the inject's inputs), the norm weight
    const u32x4* codes = is_inject ? icodes : dcodes;
    const uint16_t* sc = is_inject ? iscales : dscales;
    const uint16_t* bi = is_inject ? ibiases : dbiases;
    const u32x4 cw = __builtin_nontemporal_load(codes + (size_t)r * (G * 2) + t);
    const float s = bf16_to_f32(sc[(size_t)r * G + (t >> 1)]);
    const float b = bf16_to_f32(bi[(size_t)r * G + (t >> 1)]);
    const u32x4* rp = reinterpret_cast<const u32x4*>(raw + 32 * t);
    const u32x4* gp = reinterpret_cast<const u32x4*>(gamma + 32 * t);
    u32x4 ru[4], gu[4], ou[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { ru[i] = rp[i]; gu[i] = gp[i]; }
    float iwc = 0.0f;
    if constexpr (INJ) {
        const u32x4* op = reinterpret_cast<const u32x4*>(inj_out + (32 * t) % H);
#pragma unroll
        for (int i = 0; i < 4; ++i) ou[i] = op[i];
        iwc = inj_w[c];
    }

    float v[32];
    float ss = 0.0f, vs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w[4] = {ru[i].x, ru[i].y, ru[i].z, ru[i].w};
        const uint32_t g[4] = {gu[i].x, gu[i].y, gu[i].z, gu[i].w};
        if constexpr (INJ) {
            const uint32_t o[4] = {ou[i].x, ou[i].y, ou[i].z, ou[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = h2_bits(inject_pair(as_h2(w[k]), as_h2(o[k]), iwc));
            if (blockIdx.x == 0)
                reinterpret_cast<u32x4*>(hidden + 32 * t)[i] = u32x4{w[0], w[1], w[2], w[3]};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const h2 p = as_h2(w[k]);
            const float x0 = (float)p.x, x1 = (float)p.y;
            ss = __builtin_fmaf(x0, x0, ss);
            ss = __builtin_fmaf(x1, x1, ss);
            v[8 * i + 2 * k] = x0 * bf16_to_f32(g[k] & 0xFFFFu);
            v[8 * i + 2 * k + 1] = x1 * bf16_to_f32(g[k] >> 16);
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) vs += v[i];
    float pt = __builtin_fmaf(s, dot32_f32(cw, v), b * vs);

    // per-stream sums: whole 16-lane groups lie in one stream when H % 512 == 0 (DPP first);
    // otherwise every lane parks its pair
    const bool grouped = (H & 511) == 0;
    if (grouped) {
        pt = group_sum<16>(pt);
        ss = group_sum<16>(ss);
        if ((t & 15) == 0) part[t >> 4] = float2{pt, ss};
    } else {
        part[t] = float2{pt, ss};
    }
    __syncthreads();
    if (t < 64) {
        // lane c < C sums stream c's parts in order, then the C streams meet in a fixed butterfly
        float z = 0.0f;
        if (t < C) {
            const int n = grouped ? per >> 4 : per;
            const float2* pc = part + t * n;
            float P = 0.0f, S = 0.0f;
            for (int i = 0; i < n; ++i) { P += pc[i].x; S += pc[i].y; }
            const float ir = 1.0f / sqrtf(S / (float)H + eps);
            z = ir * P;
            if (row == 0) inv_rms_out[t] = ir;
        }
        if (C >= 2) z += dpp_f<DPP_XOR1>(z);
        if (C >= 4) z += dpp_f<DPP_XOR2>(z);
        if (C >= 8) z += dpp_f<DPP_HALF_MIRROR>(z);
        if (C >= 16) z += dpp_f<DPP_MIRROR>(z);
        if (t == 0) {
            z = z / (float)C;
            if (is_inject) inject_w[r] = 2.0f * sigmoid_f(z);
            else lo_out[r] = silu_f(z);
        }
    }
}

// 16 lanes per output h; LPRU = 16 / C lanes per stream row.
// NCH: chunks per lane, ceil((R / 32) / (16 / C)), rounded up to 3 or a power of two (3 at R = 320,
// C = 4); more would only issue clamped loads of chunks past the row and hold their registers.
template <int C, int NCH>
__global__ __launch_bounds__(UP_THREADS) void k_hc_up(
    const _Float16* __restrict__ raw, const uint16_t* __restrict__ gamma, int H,
    const u32x4* __restrict__ ucodes, const uint16_t* __restrict__ uscales,
    const uint16_t* __restrict__ ubiases, int R, const float* __restrict__ lo,
    const float* __restrict__ inv_rms, _Float16* __restrict__ mixed) {
    constexpr int LPRU = 16 / C;
    extern __shared__ float lds_lo[];     // [R/32][LO_PITCH]: 32-float chunks, bank-staggered
    constexpr int MAXCH = NCH;
    const int CHR = R >> 5;
    const int G = R >> 6;

    const int lane16 = threadIdx.x & 15;
    const int c = lane16 / LPRU;
    const int sub = lane16 % LPRU;
    // Blocks go to the 8 XCDs round-robin by index. Neighbouring blocks share the cache lines of
    // their rows' scales and biases (a row's are 2 R / 64 bytes), so consecutive runs of
    // positions are given to the blocks of one XCD, whose L2 then fetches each line once.
    const int nb = gridDim.x, x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int lb = x * (nb >> 3) + min(x, nb & 7) + i;
    const int h = lb * (blockDim.x >> 4) + (threadIdx.x >> 4);
    const bool live = h < H;              // whole 16-lane groups share h; no early exit before the DPP sums
    const size_t urow = (size_t)c * H + (live ? h : 0);
    const u32x4* cr = ucodes + urow * CHR;
    const uint16_t* sr = uscales + urow * G;
    const uint16_t* br = ubiases + urow * G;

    // every global load first (chunks past the row are clamped and not used), so the block costs
    // one memory round trip: this lane's code chunks with their scales and biases, the residual
    // element, its norm weight and the stream's inverse RMS, and its share of the low-rank vector
    u32x4 cc[MAXCH];
    uint32_t sv[MAXCH], bv[MAXCH];
#pragma unroll
    for (int i = 0; i < MAXCH; ++i) {
        const int ch = min(sub + LPRU * i, CHR - 1);
        cc[i] = cr[ch];                   // rows are R/32 chunks: lines are shared between lane groups
        sv[i] = sr[ch >> 1];
        bv[i] = br[ch >> 1];
    }
    const float rv = (float)raw[urow];
    const float gv = bf16_to_f32(gamma[urow]);
    const float ir = inv_rms[c];
    constexpr int LOADS = (1024 / 4 + UP_THREADS - 1) / UP_THREADS;   // f4v of lo per thread at R = 1024
    f4v lv4[LOADS];
#pragma unroll
    for (int k = 0; k < LOADS; ++k)
        lv4[k] = *reinterpret_cast<const f4v*>(lo + min((int)(threadIdx.x + UP_THREADS * k) * 4, R - 4));
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
        const int i = (threadIdx.x + UP_THREADS * k) * 4;
        if (i < R) *reinterpret_cast<f4v*>(lds_lo + (i >> 5) * LO_PITCH + (i & 31)) = lv4[k];
    }
    __syncthreads();

    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXCH; ++i) {
        const int ch = sub + LPRU * i;
        if (ch < CHR) {
            const f4v* lp = reinterpret_cast<const f4v*>(lds_lo + ch * LO_PITCH);
            float lv[32];
            float ls = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f4v t = lp[q];
                lv[4 * q] = t.x; lv[4 * q + 1] = t.y; lv[4 * q + 2] = t.z; lv[4 * q + 3] = t.w;
                ls += (t.x + t.y) + (t.z + t.w);
            }
            const float d = dot32_f32(cc[i], lv);
            acc = __builtin_fmaf(bf16_to_f32(sv[i]), d, acc);
            acc = __builtin_fmaf(bf16_to_f32(bv[i]), ls, acc);
        }
    }
    acc = group_sum<LPRU>(acc);
    const float n = rv * ir * gv;
    const float p = group_sum<16, LPRU>(sigmoid_f(acc) * n);     // over the C streams
    if (lane16 == 0 && live) mixed[h] = (_Float16)(p / (float)C);
}

// wide[c*H + h] = fp16(wide + out[h] * w[c]); 8 elements per thread, H % 8 == 0.
__global__ __launch_bounds__(256) void k_hc_inject(_Float16* __restrict__ wide,
                                                   const _Float16* __restrict__ out,
                                                   const float* __restrict__ w, int C, int H) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;   // 8-element chunk
    if (i >= (C * H) >> 3) return;
    const int e0 = i << 3;
    const float g = w[e0 / H];
    const int h0 = e0 % H;
    u32x4 a = *reinterpret_cast<const u32x4*>(wide + e0);
    const u32x4 o = *reinterpret_cast<const u32x4*>(out + h0);
    uint32_t av[4] = {a.x, a.y, a.z, a.w};
    const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) av[k] = h2_bits(inject_pair(as_h2(av[k]), as_h2(ov[k]), g));
    a = u32x4{av[0], av[1], av[2], av[3]};
    *reinterpret_cast<u32x4*>(wide + e0) = a;
}

template <int C>
void launch_up(dim3 g, int block, size_t lds, hipStream_t s, const _Float16* rw, const uint16_t* gm, int H,
               const u32x4* uc, const uint16_t* us, const uint16_t* ub, int R, const float* lo, const float* inv_rms,
               _Float16* mx) {
    constexpr int LPRU = 16 / C;
    const int need = ((R >> 5) + LPRU - 1) / LPRU;
    if (need <= 1) hipLaunchKernelGGL((k_hc_up<C, 1>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
    else if (need <= 2) hipLaunchKernelGGL((k_hc_up<C, 2>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
    else if (need <= 3) hipLaunchKernelGGL((k_hc_up<C, 3>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
    else if (need <= 4) hipLaunchKernelGGL((k_hc_up<C, 4>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
    else if (need <= 8) hipLaunchKernelGGL((k_hc_up<C, (8 < 32 / LPRU ? 8 : 32 / LPRU)>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
    else if (need <= 16) hipLaunchKernelGGL((k_hc_up<C, (16 < 32 / LPRU ? 16 : 32 / LPRU)>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
    else hipLaunchKernelGGL((k_hc_up<C, 32 / LPRU>), g, dim3(block), lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx);
}

}  // namespace

size_t dhp_hc_ws(int32_t C, int32_t R) {
    (void)C;
    const size_t b = (size_t)(R + DHP_HC_MAX_C) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

// The read of residual `raw`; with inj_out set, the residual is first formed as
// fp16(raw + inj_out[h] * inj_w[c]) and stored to `hidden` (the inject fused in front), and the
// read runs on those values.
int launch_hc_read_impl(const void* raw, const void* gamma, int C, int H, float eps, const dhp_int4* down,
                        const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w, void* ws,
                        hipStream_t s, const void* inj_out, const float* inj_w, void* hidden) {
    const int R = down->rows;
    float* lo = static_cast<float*>(ws);
    float* inv_rms = lo + R;
    const int rows = R + (inject ? C : 0);
    const int threads = (C * H) / 32;
    const auto* rin = static_cast<const _Float16*>(raw);
    const auto* gm = static_cast<const uint16_t*>(gamma);
    const auto* dc = static_cast<const u32x4*>(down->codes);
    const auto* ds = static_cast<const uint16_t*>(down->scales);
    const auto* db = static_cast<const uint16_t*>(down->biases);
    const auto* ic = inject ? static_cast<const u32x4*>(inject->codes) : nullptr;
    const auto* is = inject ? static_cast<const uint16_t*>(inject->scales) : nullptr;
    const auto* ib = inject ? static_cast<const uint16_t*>(inject->biases) : nullptr;
    const auto* io = static_cast<const _Float16*>(inj_out);
    auto* hid = static_cast<_Float16*>(hidden);
    if (inj_out)
        hipLaunchKernelGGL(k_hc_down<true>, dim3(rows), dim3(threads), 0, s, rin, gm, C, H, eps, dc, ds, db, R, ic,
                           is, ib, io, inj_w, hid, lo, inv_rms, inject_w);
    else
        hipLaunchKernelGGL(k_hc_down<false>, dim3(rows), dim3(threads), 0, s, rin, gm, C, H, eps, dc, ds, db, R, ic,
                           is, ib, io, inj_w, hid, lo, inv_rms, inject_w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "hc_down launch: %s", hipGetErrorString(e));

    const int block = UP_THREADS;          // 4 outputs per block
    const dim3 g((unsigned)((H + 3) / 4));
    const size_t lds = (size_t)(R / 32) * LO_PITCH * sizeof(float);
    const auto* rw = inj_out ? static_cast<const _Float16*>(hidden) : rin;   // the residual the read saw
    const auto* uc = static_cast<const u32x4*>(up->codes);
    const auto* us = static_cast<const uint16_t*>(up->scales);
    const auto* ub = static_cast<const uint16_t*>(up->biases);
    auto* mx = static_cast<_Float16*>(mixed);
    switch (C) {
        case 1: launch_up<1>(g, block, lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx); break;
        case 2: launch_up<2>(g, block, lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx); break;
        case 4: launch_up<4>(g, block, lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx); break;
        case 8: launch_up<8>(g, block, lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx); break;
        case 16: launch_up<16>(g, block, lds, s, rw, gm, H, uc, us, ub, R, lo, inv_rms, mx); break;
        default: return dhp_fail(DHP_ERR_UNSUPPORTED, "C=%d", C);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "hc_up launch: %s", hipGetErrorString(e));
    return DHP_OK;
}

int launch_hc_read(const void* raw, const void* gamma, int C, int H, float eps, const dhp_int4* down,
                   const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w,
                   void* ws, hipStream_t s) {
    return launch_hc_read_impl(raw, gamma, C, H, eps, down, up, inject, mixed, inject_w, ws, s, nullptr, nullptr,
                               nullptr);
}

int launch_hc_inject_read(const void* prev, const void* out, const float* w, void* hidden, const void* gamma, int C,
                          int H, float eps, const dhp_int4* down, const dhp_int4* up, const dhp_int4* inject,
                          void* mixed, float* inject_w, void* ws, hipStream_t s) {
    return launch_hc_read_impl(prev, gamma, C, H, eps, down, up, inject, mixed, inject_w, ws, s, out, w, hidden);
}

int launch_hc_inject(void* wide, const void* out, const float* w, int C, int H, hipStream_t s) {
    const int chunks = (C * H) / 8;
    hipLaunchKernelGGL(k_hc_inject, dim3((chunks + 255) / 256), dim3(256), 0, s,
                       static_cast<_Float16*>(wide), static_cast<const _Float16*>(out), w, C, H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "hc_inject launch: %s", hipGetErrorString(e));
    return DHP_OK;
}
