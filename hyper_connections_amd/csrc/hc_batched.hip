// The hyper-connection read and inject for the m tokens of a chunked-prefill micro-batch.
//
// "src/families/qwen4/hc.rs", encode_hyper_connection: the same read as the decode path, per
// token, with each token's inject gate in a row of its own (inside a micro-batch a later token's
// gate must not overwrite an earlier one's before its inject reads it); "src/families/qwen4/
// mod.rs", section Hyper-connections, for the steps. With m rows the three low-rank projections
// are small dense contractions, so they run on the matrix cores through the batched GEMM arm
// instead of m GEMVs:
//
//  k_hcb_norm   : one block per (token, stream): the stream's RMS, then normed = raw / rms *
//                 hc_norm in fp32, stored once as fp16 (the GEMM operand)          -> [m][C*H]
//  GEMM down    : normed . down^T, split-K (K = C*H is long, R is short: 16 splits give the
//   + inject      matrix cores enough blocks), fp32 partials                    -> [16][m][R]
//                 and, in the same launch, normed . inject^T split the same way  -> [16][m][C]
//  k_hcb_act    : the partials summed in split order; lo = silu(. / C) (fp16, the next GEMM
//                 operand); inject_w = 2 sigmoid(. / C)
//  GEMM up      : lo . up^T; at C = 4 past 32 tokens its epilogue does the mix below (a block
//                 takes 16 positions of each stream), otherwise fp32 out          -> [m][C*H]
//  k_hcb_mix    : mixed = mean over the C streams of sigmoid(up) * normed             -> [m][H]
//
// The inject is 8 fp16 elements per thread over the m rows, each row with its own gate.
// Results match the per-token read within the tolerance, not bit for bit: normed and lo are
// rounded to fp16 here (the matrix cores' operands), where the decode read keeps them fp32.
#include "dhp_internal.hpp"

#include <math.h>

namespace {

size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }

constexpr int KSPLIT = 16;         // divides C*H/64 for every supported shape (C*H % 2048 == 0)

struct HcbWs {
    size_t normed, lo_pre, lo, ipre, upre, total;
};

HcbWs hcb_ws(int m, int C, int H, int R) {
    HcbWs w;
    const size_t wide = (size_t)C * H;
    w.normed = 0;
    w.lo_pre = w.normed + a256((size_t)m * wide * 2);
    w.lo = w.lo_pre + a256((size_t)KSPLIT * m * R * 4);
    w.ipre = w.lo + a256((size_t)m * R * 2);
    w.upre = w.ipre + a256((size_t)KSPLIT * m * C * 4);
    w.total = w.upre + a256((size_t)m * wide * 4);
    return w;
}

// One block per (token, stream): H / 8 eight-element chunks, NCH per thread, all loaded before
// the reduction (NCH = ceil(H / 2048): two for H = 2560).
constexpr int NORM_MAX_CHUNKS = 16;         // per thread: H <= 256 * 8 * 16 = 32768
template <int NCH>
__global__ __launch_bounds__(256) void k_hcb_norm(const _Float16* __restrict__ raw, const uint16_t* __restrict__ gamma,
                                                  _Float16* __restrict__ normed, int C, int H, float eps) {
    __shared__ float wsum[4];
    const int m = blockIdx.x, c = blockIdx.y;
    const size_t base = ((size_t)m * C + c) * H;           // row m, stream c
    const int n8 = H >> 3;
    u32x4 v[NCH], g[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int i = min((int)threadIdx.x + 256 * k, n8 - 1);
        v[k] = *reinterpret_cast<const u32x4*>(raw + base + 8 * i);
        g[k] = *reinterpret_cast<const u32x4*>(gamma + (size_t)c * H + 8 * i);
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        if ((int)threadIdx.x + 256 * k < n8) {
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const h2 x = as_h2(w[q]);
                ss = __builtin_fmaf((float)x.x, (float)x.x, ss);
                ss = __builtin_fmaf((float)x.y, (float)x.y, ss);
            }
        }
    }
    ss = group_sum<64>(ss);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)H + eps);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int i = (int)threadIdx.x + 256 * k;
        if (i < n8) {
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
            const uint32_t gw[4] = {g[k].x, g[k].y, g[k].z, g[k].w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const h2 x = as_h2(w[q]);
                const h2 r = {(_Float16)((float)x.x * inv * bf16_to_f32(gw[q] & 0xFFFFu)),
                              (_Float16)((float)x.y * inv * bf16_to_f32(gw[q] >> 16))};
                o[q] = h2_bits(r);
            }
            *reinterpret_cast<u32x4*>(normed + base + 8 * i) = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
}

__global__ __launch_bounds__(256) void k_hcb_act(const float* __restrict__ lo_pre, _Float16* __restrict__ lo,
                                                 const float* __restrict__ ipre, float* __restrict__ inject_w,
                                                 int n_lo, int n_iw, float inv_c) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n_lo) {
        float z = 0.0f;
#pragma unroll
        for (int k = 0; k < KSPLIT; ++k) z += lo_pre[(size_t)k * n_lo + i];
        lo[i] = (_Float16)silu_f(z * inv_c);
    } else if (i - n_lo < n_iw) {
        const int j = i - n_lo;
        float z = 0.0f;
#pragma unroll
        for (int k = 0; k < KSPLIT; ++k) z += ipre[(size_t)k * n_iw + j];
        inject_w[j] = 2.0f * sigmoid_f(z * inv_c);
    }
}

__global__ __launch_bounds__(256) void k_hcb_mix(const float* __restrict__ upre, const _Float16* __restrict__ normed,
                                                 _Float16* __restrict__ mixed, int m, int C, int H) {
    const int i = blockIdx.x * 256 + threadIdx.x;          // (token, h)
    if (i >= m * H) return;
    const int t = i / H, h = i - t * H;
    const size_t row = (size_t)t * C * H + h;
    float p = 0.0f;
    for (int c = 0; c < C; ++c) p += sigmoid_f(upre[row + (size_t)c * H]) * (float)normed[row + (size_t)c * H];
    mixed[i] = (_Float16)(p / (float)C);
}

// wide[t][c*H + h] = fp16(wide + out[t][h] * w[t][c]); 8 elements per thread.
__global__ __launch_bounds__(256) void k_hcb_inject(_Float16* __restrict__ wide, const _Float16* __restrict__ out,
                                                    const float* __restrict__ w, int m, int C, int H) {
    const int i = blockIdx.x * 256 + threadIdx.x;          // 8-element chunk over [m][C*H]
    const int per = (C * H) >> 3;
    if (i >= m * per) return;
    const int t = i / per, e0 = (i - t * per) << 3;
    const float g = w[(size_t)t * C + e0 / H];
    const int h0 = e0 % H;
    _Float16* wp = wide + (size_t)t * C * H + e0;
    const u32x4 a = *reinterpret_cast<const u32x4*>(wp);
    const u32x4 o = *reinterpret_cast<const u32x4*>(out + (size_t)t * H + h0);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, ov[4] = {o.x, o.y, o.z, o.w};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = h2_bits(inject_pair(as_h2(av[k]), as_h2(ov[k]), g));
    *reinterpret_cast<u32x4*>(wp) = u32x4{r[0], r[1], r[2], r[3]};
}

template <int NCH>
void launch_norm_n(dim3 g, hipStream_t s, const _Float16* raw, const uint16_t* gamma, _Float16* normed, int C, int H,
                   float eps) {
    hipLaunchKernelGGL(k_hcb_norm<NCH>, g, dim3(256), 0, s, raw, gamma, normed, C, H, eps);
}

void launch_norm(dim3 g, hipStream_t s, const _Float16* raw, const uint16_t* gamma, _Float16* normed, int C, int H,
                 float eps) {
    switch ((H / 8 + 255) / 256) {
        case 1: launch_norm_n<1>(g, s, raw, gamma, normed, C, H, eps); break;
        case 2: launch_norm_n<2>(g, s, raw, gamma, normed, C, H, eps); break;
        case 3: launch_norm_n<3>(g, s, raw, gamma, normed, C, H, eps); break;
        case 4: launch_norm_n<4>(g, s, raw, gamma, normed, C, H, eps); break;
        case 5: case 6: case 7: case 8: launch_norm_n<8>(g, s, raw, gamma, normed, C, H, eps); break;
        default: launch_norm_n<NORM_MAX_CHUNKS>(g, s, raw, gamma, normed, C, H, eps); break;
    }
}

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DHP_OK : dhp_fail(DHP_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
}

}  // namespace

size_t dhp_hc_read_batched_ws(int32_t m, int32_t C, int32_t H, int32_t R) { return hcb_ws(m, C, H, R).total; }

int launch_hc_read_batched(const void* raw, int m, const void* gamma, int C, int H, float eps, const dhp_int4* down,
                           const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w, void* ws,
                           hipStream_t s) {
    const int R = down->rows;
    const HcbWs lay = hcb_ws(m, C, H, R);
    char* b = static_cast<char*>(ws);
    _Float16* normed = reinterpret_cast<_Float16*>(b + lay.normed);
    float* lo_pre = reinterpret_cast<float*>(b + lay.lo_pre);
    _Float16* lo = reinterpret_cast<_Float16*>(b + lay.lo);
    float* ipre = reinterpret_cast<float*>(b + lay.ipre);
    float* upre = reinterpret_cast<float*>(b + lay.upre);

    launch_norm(dim3(m, C), s, static_cast<const _Float16*>(raw), static_cast<const uint16_t*>(gamma), normed, C, H,
                eps);
    int rc = launch_status("hc norm");
    // the down and inject projections share the normed rows and K: one launch for both
    if (!rc) rc = launch_gemm_mfma_splitk(down, normed, m, lo_pre, KSPLIT, s, inject, inject ? ipre : nullptr);
    if (rc) return rc;
    const int n_lo = m * R, n_iw = inject ? m * C : 0;
    hipLaunchKernelGGL(k_hcb_act, dim3((n_lo + n_iw + 255) / 256), dim3(256), 0, s, lo_pre, lo, ipre, inject_w,
                       n_lo, n_iw, 1.0f / (float)C);
    rc = launch_status("hc act");
    if (rc) return rc;
    // four streams and a chunk of more than 32 tokens: the up GEMM's epilogue does the stream mix
    if (dhp_gemm_upmix_fits(up, m, C, H)) return launch_gemm_mfma_upmix(up, lo, m, normed, mixed, H, s);
    rc = launch_gemm_mfma(up, lo, m, upre, 1, nullptr, nullptr, 0, s);
    if (rc) return rc;
    hipLaunchKernelGGL(k_hcb_mix, dim3((m * H + 255) / 256), dim3(256), 0, s, upre, normed,
                       static_cast<_Float16*>(mixed), m, C, H);
    return launch_status("hc mix");
}

int launch_hc_inject_batched(void* wide, int m, const void* out, const float* w, int C, int H, hipStream_t s) {
    const int chunks = m * ((C * H) >> 3);
    hipLaunchKernelGGL(k_hcb_inject, dim3((chunks + 255) / 256), dim3(256), 0, s, static_cast<_Float16*>(wide),
                       static_cast<const _Float16*>(out), w, m, C, H);
    return launch_status("hc inject");
}
