// Hyper-connection read (grouped RMS norm, low-rank mix, inject gate) and inject add.
//
// "src/families/qwen4/mod.rs" (turbospark-runtime 0.3.0), section Hyper-connections, and
// "src/families/qwen4/hc.rs", encode_hyper_connection. The pages run one dispatch per
// step (norm, down GEMV, scale by 1/C, SiLU, up GEMV, sigmoid, mix, inject GEMV, scale,
// sigmoid, scale by 2). Here the read is two kernels:
//
//  k_hc_down : one block per output row of the down projection (R rows) and of the inject
//              projection (C rows). Every block recomputes the C stream RMS values from the
//              20 KB residual (an L2 hit after the first block), normalizes its own 32-wide
//              slice in registers, and reduces one dot product over the whole C*H input:
//              lane t owns input positions 32t..32t+31, so the block is C*H/32 lanes wide.
//              The epilogue applies the 1/C, then SiLU (down rows) or 2*sigmoid (inject rows).
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

// raw, gamma: the C*H stream; one block per projection row (down rows first, then inject rows).
__global__ __launch_bounds__(HC_MAX_THREADS) void k_hc_down(
    const _Float16* __restrict__ raw, const uint16_t* __restrict__ gamma, int C, int H, float eps,
    const u32x4* __restrict__ dcodes, const uint16_t* __restrict__ dscales,
    const uint16_t* __restrict__ dbiases, int R, const u32x4* __restrict__ icodes,
    const uint16_t* __restrict__ iscales, const uint16_t* __restrict__ ibiases,
    float* __restrict__ lo_out, float* __restrict__ inv_rms_out, float* __restrict__ inject_w) {
    __shared__ float part[HC_MAX_THREADS];
    __shared__ float inv_rms[DHP_HC_MAX_C];
    __shared__ float wsum[HC_MAX_THREADS / 64];

    const int t = threadIdx.x;            // chunk index, input positions 32t .. 32t+31
    const int CH = (C * H) >> 5;          // == blockDim.x
    const int G = (C * H) >> 6;
    const int row = blockIdx.x;
    const bool is_inject = row >= R;
    const int r = is_inject ? row - R : row;

    // this block's weight slice first, so it is in flight during the norm
    const u32x4* codes = is_inject ? icodes : dcodes;
    const uint16_t* sc = is_inject ? iscales : dscales;
    const uint16_t* bi = is_inject ? ibiases : dbiases;
    const u32x4 c = __builtin_nontemporal_load(codes + (size_t)r * CH + t);
    const float s = bf16_to_f32(sc[(size_t)r * G + (t >> 1)]);
    const float b = bf16_to_f32(bi[(size_t)r * G + (t >> 1)]);

    // residual slice and its squares
    float v[32];
    {
        const u32x4* rp = reinterpret_cast<const u32x4*>(raw + 32 * t);
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 u = rp[i];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const h2 p = as_h2(w[k]);
                v[8 * i + 2 * k] = (float)p.x;
                v[8 * i + 2 * k + 1] = (float)p.y;
                ss = __builtin_fmaf(v[8 * i + 2 * k], v[8 * i + 2 * k], ss);
                ss = __builtin_fmaf(v[8 * i + 2 * k + 1], v[8 * i + 2 * k + 1], ss);
            }
        }
        // a stream's H/32 chunks are whole 16-lane groups when H % 512 == 0: sum within each
        // group first (DPP), leaving H/512 partials per stream
        if ((H & 511) == 0) {
            ss = group_sum<16>(ss);
            if ((t & 15) == 0) part[t >> 4] = ss;
        } else {
            part[t] = ss;
        }
    }
    __syncthreads();
    const int per = H >> 5;               // chunks per stream
    if (t < C) {
        float acc = 0.0f;
        if ((H & 511) == 0) {
            const int pg = per >> 4;      // 16-lane groups per stream
            for (int i = 0; i < pg; ++i) acc += part[t * pg + i];
        } else {
            for (int i = 0; i < per; ++i) acc += part[t * per + i];
        }
        inv_rms[t] = 1.0f / sqrtf(acc / (float)H + eps);
    }
    __syncthreads();

    // normalized slice (direct-scale weight), its dot with the codes, and its sum
    const float ir = inv_rms[t / per];
    {
        const u32x4* gp = reinterpret_cast<const u32x4*>(gamma + 32 * t);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 u = gp[i];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[8 * i + 2 * k] = v[8 * i + 2 * k] * ir * bf16_to_f32(w[k] & 0xFFFFu);
                v[8 * i + 2 * k + 1] = v[8 * i + 2 * k + 1] * ir * bf16_to_f32(w[k] >> 16);
            }
        }
    }
    float xs = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) xs += v[i];
    float acc = __builtin_fmaf(s, dot32_f32(c, v), b * xs);

    acc = group_sum<64>(acc);
    if ((t & 63) == 0) wsum[t >> 6] = acc;
    __syncthreads();
    if (t == 0) {
        float tot = 0.0f;
        const int nw = (CH + 63) >> 6;
        for (int w = 0; w < nw; ++w) tot += wsum[w];
        const float z = tot / (float)C;
        if (is_inject) inject_w[r] = 2.0f * sigmoid_f(z);
        else lo_out[r] = silu_f(z);
        if (row == 0)
            for (int k = 0; k < C; ++k) inv_rms_out[k] = inv_rms[k];
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
    const int h = blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4);
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
    for (int k = 0; k < 4; ++k) {
        const h2 x = as_h2(av[k]), y = as_h2(ov[k]);
        h2 r;
        r.x = (_Float16)__builtin_fmaf((float)y.x, g, (float)x.x);
        r.y = (_Float16)__builtin_fmaf((float)y.y, g, (float)x.y);
        av[k] = h2_bits(r);
    }
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

int launch_hc_read(const void* raw, const void* gamma, int C, int H, float eps, const dhp_int4* down,
                   const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w,
                   void* ws, hipStream_t s) {
    const int R = down->rows;
    float* lo = static_cast<float*>(ws);
    float* inv_rms = lo + R;
    const int rows = R + (inject ? C : 0);
    const int threads = (C * H) / 32;
    hipLaunchKernelGGL(k_hc_down, dim3(rows), dim3(threads), 0, s,
                       static_cast<const _Float16*>(raw), static_cast<const uint16_t*>(gamma), C, H, eps,
                       static_cast<const u32x4*>(down->codes), static_cast<const uint16_t*>(down->scales),
                       static_cast<const uint16_t*>(down->biases), R,
                       inject ? static_cast<const u32x4*>(inject->codes) : nullptr,
                       inject ? static_cast<const uint16_t*>(inject->scales) : nullptr,
                       inject ? static_cast<const uint16_t*>(inject->biases) : nullptr, lo, inv_rms,
                       inject_w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "hc_down launch: %s", hipGetErrorString(e));

    const int block = UP_THREADS;          // 4 outputs per block
    const dim3 g((unsigned)((H + 3) / 4));
    const size_t lds = (size_t)(R / 32) * LO_PITCH * sizeof(float);
    const auto* rw = static_cast<const _Float16*>(raw);
    const auto* gm = static_cast<const uint16_t*>(gamma);
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

int launch_hc_inject(void* wide, const void* out, const float* w, int C, int H, hipStream_t s) {
    const int chunks = (C * H) / 8;
    hipLaunchKernelGGL(k_hc_inject, dim3((chunks + 255) / 256), dim3(256), 0, s,
                       static_cast<_Float16*>(wide), static_cast<const _Float16*>(out), w, C, H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "hc_inject launch: %s", hipGetErrorString(e));
    return DHP_OK;
}
