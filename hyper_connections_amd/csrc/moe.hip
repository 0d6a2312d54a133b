// Routed mixture-of-experts decode for one token: router GEMV, on-device top-k with softmax
// over the selected experts, phase 1 (gate/up GEMV + silu(gate)*up), phase 2 (down GEMV +
// weighted k-way reduce) and the sigmoid-gated shared expert.
//
// "src/families/qwen4/mod.rs" (turbospark-runtime 0.3.0), section MoE; "src/families/qwen/
// state.rs", struct RealQwenState (fp32 router logits, unit router scales, gated shared
// expert); "src/real_forward.rs", module doc (phase-1 gate_up_act and phase-2 down_reduce
// kernels, with the router logits read back to the host for top-k between two command
// buffers). Here nothing returns to the host: three kernels on one stream.
//
//  k_moe_router : one wave per router row (fp32 logits into the workspace), one wave for the
//                 shared expert's scalar gate logit, and quarter-waves running the shared
//                 expert's gate/up pairs, which need no routing decision.
//  k_moe_phase1 : every block re-derives the top-k from the E logits (a handful of wave
//                 maxima, cheaper than another launch), then its quarter-waves run one
//                 (selected expert, row) pair each: gate and up rows against register-resident
//                 activations, act = silu(gate) * up in fp32. Block 0 writes ids and weights.
//  k_moe_phase2 : 16 lanes per output element walk the down rows of the selected experts and
//                 the shared expert (K = inter) against the fp32 activations staged in LDS,
//                 four waves splitting the experts, each expert's partial weighted by its
//                 softmax weight; the shared part is scaled by sigmoid(g) and both halves meet
//                 in one fp16 rounding.
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

namespace {

constexpr int LPR = 16;
constexpr int MAX_E = 1024;

struct MoeArgs {
    const _Float16* x;
    const void* router;
    int router_f32;
    const uint16_t* sgate_row;
    // routed experts: first tensor and byte strides
    const uint8_t* g_codes; const uint8_t* g_scales; const uint8_t* g_biases;
    const uint8_t* u_codes; const uint8_t* u_scales; const uint8_t* u_biases;
    const uint8_t* d_codes; const uint8_t* d_scales; const uint8_t* d_biases;
    long long gu_cstride, gu_sstride;     // gate and up share strides (same shapes)
    long long u_cstride, u_sstride;
    long long d_cstride, d_sstride;
    // shared expert
    const u32x4* sg_codes; const uint16_t* sg_scales; const uint16_t* sg_biases;
    const u32x4* su_codes; const uint16_t* su_scales; const uint16_t* su_biases;
    const u32x4* sd_codes; const uint16_t* sd_scales; const uint16_t* sd_biases;
    int E, hidden, inter, top_k, boundary;
    float* logits;     // ws [E]
    float* gate_logit; // ws [1]
    float* act;        // ws [(top_k + 1) * inter]; slot top_k is the shared expert
    _Float16* out;
    int32_t* ids;
    float* weights;
};

// Registers of one (gate row, up row) pair for the 16-lane group whose lane index is j.
template <int CPL>
struct PairRegs {
    u32x4 cg[CPL], cu[CPL];
    uint32_t sg[CPL], bg[CPL], su[CPL], bu[CPL];
};

// Issue the code/scale/bias loads of gate row `row` and up row `row` (K = hidden = 512 * CPL).
template <int CPL>
DHP_DEV void load_pair(PairRegs<CPL>& p, const u32x4* gc, const uint16_t* gs, const uint16_t* gb,
                       const u32x4* uc, const uint16_t* us, const uint16_t* ub, int row, int j) {
    constexpr int CH = LPR * CPL;
    constexpr int G = CH / 2;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = j + LPR * i;
        p.cg[i] = __builtin_nontemporal_load(gc + (size_t)row * CH + ch);
        p.cu[i] = __builtin_nontemporal_load(uc + (size_t)row * CH + ch);
        p.sg[i] = gs[(size_t)row * G + (ch >> 1)];
        p.bg[i] = gb[(size_t)row * G + (ch >> 1)];
        p.su[i] = us[(size_t)row * G + (ch >> 1)];
        p.bu[i] = ub[(size_t)row * G + (ch >> 1)];
    }
}

// silu(gate . x) * (up . x), the same value in every lane of the 16-lane group. The chunk dots
// use the raw code form (see dot32_f16_raw) with the activations' per-chunk corrections nc.
template <int CPL>
DHP_DEV float pair_act(const PairRegs<CPL>& p, const h2 (*xp)[16], const float* xs, const float* nc) {
    const NibConsts nk = nib_consts();
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        ag = __builtin_fmaf(bf16_to_f32(p.sg[i]), dot32_f16_raw(p.cg[i], xp[i], nc[i], nk), ag);
        ag = __builtin_fmaf(bf16_to_f32(p.bg[i]), xs[i], ag);
        au = __builtin_fmaf(bf16_to_f32(p.su[i]), dot32_f16_raw(p.cu[i], xp[i], nc[i], nk), au);
        au = __builtin_fmaf(bf16_to_f32(p.bu[i]), xs[i], au);
    }
    ag = group_sum<LPR>(ag);
    au = group_sum<LPR>(au);
    return silu_f(ag) * au;
}

// fp32 dot of one bf16 or fp32 row of length hidden = 512 * CPL with the fp16 activations, one
// wave. Every load of the row is issued before the first product, so the row costs one memory
// round trip.
template <int CPL>
DHP_DEV float wave_row_dot(const void* row, int f32, const _Float16* x) {
    const int lane = threadIdx.x & 63;
    float acc = 0.0f;
    if (!f32) {
        const u32x4* r = static_cast<const u32x4*>(row);          // 8 bf16 per chunk, CPL per lane
        u32x4 w[CPL], xv[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            w[i] = __builtin_nontemporal_load(r + lane + 64 * i);
            xv[i] = *reinterpret_cast<const u32x4*>(x + 8 * (lane + 64 * i));
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            const uint32_t xx[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const h2 xh = as_h2(xx[k]);
                acc = __builtin_fmaf(bf16_to_f32(ww[k] & 0xFFFFu), (float)xh.x, acc);
                acc = __builtin_fmaf(bf16_to_f32(ww[k] >> 16), (float)xh.y, acc);
            }
        }
    } else {
        const f4v* r = static_cast<const f4v*>(row);               // 4 fp32 per chunk, 2 CPL per lane
        f4v w[2 * CPL];
        uint2 xv[2 * CPL];
#pragma unroll
        for (int i = 0; i < 2 * CPL; ++i) {
            w[i] = __builtin_nontemporal_load(r + lane + 64 * i);
            xv[i] = *reinterpret_cast<const uint2*>(x + 4 * (lane + 64 * i));
        }
#pragma unroll
        for (int i = 0; i < 2 * CPL; ++i) {
            const h2 x0 = as_h2(xv[i].x), x1 = as_h2(xv[i].y);
            acc = __builtin_fmaf(w[i].x, (float)x0.x, acc);
            acc = __builtin_fmaf(w[i].y, (float)x0.y, acc);
            acc = __builtin_fmaf(w[i].z, (float)x1.x, acc);
            acc = __builtin_fmaf(w[i].w, (float)x1.y, acc);
        }
    }
    return group_sum<64>(acc);
}

template <int CPL>
DHP_DEV void load_x_regs(const _Float16* x, int j, h2 (*xp)[16], float* xs, float* nc) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) xs[i] = load_x32_raw(x + (size_t)(j + LPR * i) * 32, xp[i], nc[i]);
}

// Blocks [0, E): router rows. Block E: shared gate logit. Blocks after: 4 shared pairs each.
template <int CPL>
__global__ __launch_bounds__(64) void k_moe_router(MoeArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    if (b < a.E) {
        const size_t rb = (size_t)a.hidden * (a.router_f32 ? 4 : 2);
        const float v = wave_row_dot<CPL>(static_cast<const uint8_t*>(a.router) + rb * b, a.router_f32, a.x);
        if (lane == 0) a.logits[b] = v;
        return;
    }
    if (b == a.E) {
        const float v = wave_row_dot<CPL>(a.sgate_row, 0, a.x);
        if (lane == 0) a.gate_logit[0] = v;
        return;
    }
    const int j = lane % LPR;
    const int row = (b - a.E - 1) * 4 + lane / LPR;
    const bool live = row < a.inter;      // 16-lane groups share a row; all lanes stay for the DPP sums
    PairRegs<CPL> p;
    load_pair<CPL>(p, a.sg_codes, a.sg_scales, a.sg_biases, a.su_codes, a.su_scales, a.su_biases,
                   live ? row : 0, j);
    h2 xp[CPL][16];
    float xs[CPL], nc[CPL];
    load_x_regs<CPL>(a.x, j, xp, xs, nc);
    const float v = pair_act<CPL>(p, xp, xs, nc);
    if (j == 0 && live) a.act[(size_t)a.top_k * a.inter + row] = v;
}

// Top-k by one wave. Every logit becomes an unsigned word that orders like the float (a NaN
// ranks as -inf; -0 is folded into +0, they compare equal) and lane l holds the words of the
// PER consecutive experts l*PER + i, so a lower lane always means lower expert indices. Each
// round takes the wave-wide maximum word; the lowest lane holding it gives up its entry (the
// lowest index among equal words), and the next round starts over.
// Padding entries (e >= E) hold 0, below every real logit (the -inf word is 0x007FFFFF).
DHP_DEV uint32_t order_word(float l) {
    l = (l == l) ? l + 0.0f : -INFINITY;
    const uint32_t u = __builtin_bit_cast(uint32_t, l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DHP_DEV float order_word_value(uint32_t u) {
    return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Wave-wide maximum, in every lane: DPP within each 16-lane row, then the gfx950 row swap
// (odd rows against even rows) and half swap (upper 32 lanes against lower 32).
DHP_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<DPP_XOR1>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_XOR2>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_HALF_MIRROR>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_MIRROR>((int)v));
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((uint32_t)r[0], (uint32_t)r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)h[0], (uint32_t)h[1]);
}

// The logits a lane ranks: PER consecutive ones from lane * PER, in whole 16-byte loads clamped
// to the last full vector (the buffer must be readable up to index 4 * ((E - 1) / 4) + 3).
template <int PER>
struct TopkIn {
    u32x4 v[PER / 4];
};
template <int PER>
DHP_DEV void topk_load(TopkIn<PER>& t, const float* logits, int E) {
    static_assert(PER % 4 == 0, "whole 16-byte loads");
    const int lane = threadIdx.x & 63;
    const int last4 = ((E - 1) >> 2) << 2;
#pragma unroll
    for (int q = 0; q < PER / 4; ++q)
        t.v[q] = *reinterpret_cast<const u32x4*>(logits + min(lane * PER + 4 * q, last4));
}

// The first `rounds` entries of the top-k of the E logits (E <= 64 * PER); every lane returns
// the same ids and values.
template <int PER>
DHP_DEV void wave_topk(TopkIn<PER>& t, int E, int rounds, int* ids, float* vals) {
    const int lane = threadIdx.x & 63;
    uint32_t w[PER];
    int ix[PER];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t u = t.v[q][c];
            asm volatile("" : "+v"(u));  // every element is live: the loads stay whole vectors
            w[4 * q + c] = order_word(__builtin_bit_cast(float, u));
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        w[i] = (lane * PER + i < E) ? w[i] : 0u;
        ix[i] = i;
    }
    if constexpr (PER <= 4) {
        // sort each lane's entries: adjacent exchanges on a strict comparison keep equal words
        // in index order
#pragma unroll
        for (int p = 0; p < PER - 1; ++p) {
#pragma unroll
            for (int q = 0; q < PER - 1 - p; ++q) {
                const bool sw = w[q + 1] > w[q];
                const uint32_t w0 = w[q], w1 = w[q + 1];
                const int i0 = ix[q], i1 = ix[q + 1];
                w[q] = sw ? w1 : w0;
                w[q + 1] = sw ? w0 : w1;
                ix[q] = sw ? i1 : i0;
                ix[q + 1] = sw ? i0 : i1;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < DHP_MOE_MAX_TOP_K; ++r) {
        if (r >= rounds) break;
        if constexpr (PER <= 4) {
            const uint32_t m = wave_max_u32(w[0]);
            const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(w[0] == m));
            ids[r] = wl * PER + __builtin_amdgcn_readlane(ix[0], wl);
            vals[r] = order_word_value(m);
            const bool mine = lane == wl;
#pragma unroll
            for (int q = 0; q < PER - 1; ++q) {
                w[q] = mine ? w[q + 1] : w[q];
                ix[q] = mine ? ix[q + 1] : ix[q];
            }
            w[PER - 1] = mine ? 0u : w[PER - 1];
        } else {
            uint32_t best = w[0];
#pragma unroll
            for (int i = 1; i < PER; ++i) best = max(best, w[i]);
            const uint32_t m = wave_max_u32(best);
            const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(best == m));
            int first = PER - 1;
#pragma unroll
            for (int i = PER - 2; i >= 0; --i) first = (w[i] == m) ? i : first;
            ids[r] = wl * PER + __builtin_amdgcn_readlane(first, wl);
            vals[r] = order_word_value(m);
            const bool mine = lane == wl;
#pragma unroll
            for (int i = 0; i < PER; ++i) w[i] = (mine && i == first) ? 0u : w[i];
        }
    }
}

template <int CPL, int PER>
__global__ __launch_bounds__(64) void k_moe_phase1(MoeArgs a) {
    const int lane = threadIdx.x;
    const int j = lane % LPR;
    TopkIn<PER> tin;
    topk_load<PER>(tin, a.logits, a.E);    // the routing decision waits on these: issue first
    h2 xp[CPL][16];
    float xs[CPL], nc[CPL];
    load_x_regs<CPL>(a.x, j, xp, xs, nc);  // independent of routing

    // a block only needs the ranks up to its last (slot, row) pair; block 0 also needs all
    // top_k of them for the softmax weights
    const int last_pair = min((int)blockIdx.x * 4 + 3, a.top_k * a.inter - 1);
    const int rounds = (blockIdx.x == 0) ? a.top_k : last_pair / a.inter + 1;
    int ids[DHP_MOE_MAX_TOP_K];
    float vals[DHP_MOE_MAX_TOP_K];
    wave_topk<PER>(tin, a.E, rounds, ids, vals);

    const int pair = blockIdx.x * 4 + lane / LPR;      // (slot, row) flattened
    const bool live = pair < a.top_k * a.inter;
    const int slot = live ? pair / a.inter : 0;
    const int row = live ? pair % a.inter : 0;
    int e = ids[0];
#pragma unroll
    for (int r = 1; r < DHP_MOE_MAX_TOP_K; ++r)
        if (r == slot) e = ids[r];
    const auto* gc = reinterpret_cast<const u32x4*>(a.g_codes + (size_t)e * a.gu_cstride);
    const auto* gs = reinterpret_cast<const uint16_t*>(a.g_scales + (size_t)e * a.gu_sstride);
    const auto* gb = reinterpret_cast<const uint16_t*>(a.g_biases + (size_t)e * a.gu_sstride);
    const auto* uc = reinterpret_cast<const u32x4*>(a.u_codes + (size_t)e * a.u_cstride);
    const auto* us = reinterpret_cast<const uint16_t*>(a.u_scales + (size_t)e * a.u_sstride);
    const auto* ub = reinterpret_cast<const uint16_t*>(a.u_biases + (size_t)e * a.u_sstride);
    PairRegs<CPL> p;
    load_pair<CPL>(p, gc, gs, gb, uc, us, ub, row, j);

    // block 0 publishes the ids and the softmax over the selected logits
    if (blockIdx.x == 0 && lane == 0) {
        float wt[DHP_MOE_MAX_TOP_K];
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < DHP_MOE_MAX_TOP_K; ++r) {
            wt[r] = (r < a.top_k) ? __expf(vals[r] - vals[0]) : 0.0f;
            sum += wt[r];
        }
#pragma unroll
        for (int r = 0; r < DHP_MOE_MAX_TOP_K; ++r) {
            if (r < a.top_k) {
                a.ids[r] = ids[r];
                a.weights[r] = wt[r] / sum;
            }
        }
    }

    const float v = pair_act<CPL>(p, xp, xs, nc);
    if (j == 0 && live) a.act[(size_t)slot * a.inter + row] = v;
}

// Phase 2. A block of four waves owns 4 * RH consecutive outputs h (16 lanes and RH outputs per
// 16-lane group, the same rows in every wave). Wave w takes expert slots w, w+4, w+8 (slot
// top_k is the shared expert): its lanes issue every code, scale and bias load of those slots
// first, the block stages the fp32 activations in LDS meanwhile, then each lane reduces its own
// chunk (K = inter; lane j takes chunks j + 16 i) of each down row. The four waves' partial sums
// meet in LDS in a fixed order, so the result does not depend on timing.
constexpr int RH = 2;
constexpr int NSLOT = DHP_MOE_MAX_TOP_K + 1;
constexpr int SLOTS_PER_WAVE = (NSLOT + 3) / 4;
constexpr int ACT_PITCH = 36;          // floats per staged 32-float activation chunk

template <int CPLD>
__global__ __launch_bounds__(256) void k_moe_phase2(MoeArgs a) {
    extern __shared__ float lds_act[];     // [(top_k + 1) * inter / 32][ACT_PITCH]
    __shared__ float part[4][2][64 * RH];  // [wave][routed, shared][lane-major partials]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int j = lane % LPR;
    const int nslot = a.top_k + 1;
    const int CH = a.inter >> 5;
    const int G = a.inter >> 6;
    const int h0 = (blockIdx.x * 4 + lane / LPR) * RH;

    // the routing weights and the shared gate logit are read up front, with the expert ids
    float wgts[SLOTS_PER_WAVE];
#pragma unroll
    for (int t = 0; t < SLOTS_PER_WAVE; ++t) {
        const int slot = wave + 4 * t;
        wgts[t] = (slot < a.top_k) ? a.weights[slot] : 1.0f;
    }
    const float gate_logit = a.gate_logit[0];

    u32x4 c[SLOTS_PER_WAVE][RH][CPLD];
    uint32_t sv[SLOTS_PER_WAVE][RH][CPLD], bv[SLOTS_PER_WAVE][RH][CPLD];
#pragma unroll
    for (int t = 0; t < SLOTS_PER_WAVE; ++t) {
        const int slot = wave + 4 * t;
        if (slot < nslot) {
            const u32x4* dc;
            const uint16_t* ds;
            const uint16_t* db;
            if (slot == a.top_k) {
                dc = a.sd_codes; ds = a.sd_scales; db = a.sd_biases;
            } else {
                const int e = a.ids[slot];
                dc = reinterpret_cast<const u32x4*>(a.d_codes + (size_t)e * a.d_cstride);
                ds = reinterpret_cast<const uint16_t*>(a.d_scales + (size_t)e * a.d_sstride);
                db = reinterpret_cast<const uint16_t*>(a.d_biases + (size_t)e * a.d_sstride);
            }
#pragma unroll
            for (int r = 0; r < RH; ++r) {
                const int h = min(h0 + r, a.hidden - 1);
#pragma unroll
                for (int i = 0; i < CPLD; ++i) {
                    const int ch = min(j + LPR * i, CH - 1);
                    c[t][r][i] = __builtin_nontemporal_load(dc + (size_t)h * CH + ch);
                    sv[t][r][i] = ds[(size_t)h * G + (ch >> 1)];
                    bv[t][r][i] = db[(size_t)h * G + (ch >> 1)];
                }
            }
        }
    }

    // stage the activations of every slot in LDS, 32-float chunks at a 36-float pitch so the 16
    // lanes of a group (one chunk each) read distinct banks; all loads are issued (clamped) before
    // the first store, so the staging costs one round trip
    constexpr int AL = (NSLOT * 512 * CPLD + 1023) / 1024;
    const int n = nslot * a.inter;
    f4v av4[AL];
#pragma unroll
    for (int k = 0; k < AL; ++k) {
        const int i = min(threadIdx.x * 4 + k * 1024, n - 4);
        av4[k] = *reinterpret_cast<const f4v*>(a.act + i);
    }
#pragma unroll
    for (int k = 0; k < AL; ++k) {
        const int i = threadIdx.x * 4 + k * 1024;
        if (i < n) *reinterpret_cast<f4v*>(lds_act + (i >> 5) * ACT_PITCH + (i & 31)) = av4[k];
    }
    __syncthreads();

    float racc[RH], sacc[RH];
#pragma unroll
    for (int r = 0; r < RH; ++r) { racc[r] = 0.0f; sacc[r] = 0.0f; }
#pragma unroll
    for (int t = 0; t < SLOTS_PER_WAVE; ++t) {
        const int slot = wave + 4 * t;
        if (slot < nslot) {
            const bool shared = slot == a.top_k;
            const float wgt = wgts[t];
            float p[RH];
#pragma unroll
            for (int r = 0; r < RH; ++r) p[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPLD; ++i) {
                const int ch = j + LPR * i;
                if (ch < CH) {
                    const f4v* ap = reinterpret_cast<const f4v*>(lds_act + (slot * CH + ch) * ACT_PITCH);
                    float av[32];
                    float xs = 0.0f;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const f4v u = ap[q];
                        av[4 * q] = u.x; av[4 * q + 1] = u.y; av[4 * q + 2] = u.z; av[4 * q + 3] = u.w;
                        xs += (u.x + u.y) + (u.z + u.w);
                    }
#pragma unroll
                    for (int r = 0; r < RH; ++r) {
                        const float d = dot32_f32(c[t][r][i], av);
                        p[r] = __builtin_fmaf(bf16_to_f32(sv[t][r][i]), d, p[r]);
                        p[r] = __builtin_fmaf(bf16_to_f32(bv[t][r][i]), xs, p[r]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RH; ++r) {
                if (shared) sacc[r] += p[r];
                else racc[r] = __builtin_fmaf(wgt, p[r], racc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RH; ++r) {
        part[wave][0][r * 64 + lane] = group_sum<LPR>(racc[r]);
        part[wave][1][r * 64 + lane] = group_sum<LPR>(sacc[r]);
    }
    __syncthreads();
    if (wave == 0) {
        const float sg = sigmoid_f(gate_logit);
#pragma unroll
        for (int r = 0; r < RH; ++r) {
            const int h = h0 + r;
            if (j == 0 && h < a.hidden) {
                const int q = r * 64 + lane;
                const float rr = (part[0][0][q] + part[1][0][q]) + (part[2][0][q] + part[3][0][q]);
                const float ss = ((part[0][1][q] + part[1][1][q]) + (part[2][1][q] + part[3][1][q])) * sg;
                float o;
                if (a.boundary) o = (float)(_Float16)rr + (float)(_Float16)ss;
                else o = rr + ss;
                a.out[h] = (_Float16)o;
            }
        }
    }
}

template <int CPL>
hipError_t launch_all(const MoeArgs& a, hipStream_t s) {
    const int shared_blocks = (a.inter + 3) / 4;
    hipLaunchKernelGGL(k_moe_router<CPL>, dim3(a.E + 1 + shared_blocks), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int pairs = a.top_k * a.inter;
    if (a.E <= 256) hipLaunchKernelGGL((k_moe_phase1<CPL, 4>), dim3((pairs + 3) / 4), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((k_moe_phase1<CPL, MAX_E / 64>), dim3((pairs + 3) / 4), dim3(64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)(a.top_k + 1) * (a.inter / 32) * ACT_PITCH * sizeof(float);
    const dim3 g2((a.hidden + 4 * RH - 1) / (4 * RH));
    if (a.inter <= 512) hipLaunchKernelGGL(k_moe_phase2<1>, g2, dim3(256), lds, s, a);
    else hipLaunchKernelGGL(k_moe_phase2<2>, g2, dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

size_t dhp_moe_ws(int32_t n_experts, int32_t top_k, int32_t inter) {
    const size_t floats = (size_t)((n_experts + 4) & ~3) + (size_t)(top_k + 1) * inter;
    return (floats * sizeof(float) + 255) & ~(size_t)255;
}

int launch_moe(const void* x, const void* router, int router_f32, const void* sgate_row,
               const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
               const dhp_int4* sg, const dhp_int4* su, const dhp_int4* sd, int top_k, int boundary,
               void* out, int32_t* ids, float* weights, void* ws, hipStream_t s) {
    MoeArgs a;
    a.x = static_cast<const _Float16*>(x);
    a.router = router;
    a.router_f32 = router_f32;
    a.sgate_row = static_cast<const uint16_t*>(sgate_row);
    a.g_codes = static_cast<const uint8_t*>(gate->first.codes);
    a.g_scales = static_cast<const uint8_t*>(gate->first.scales);
    a.g_biases = static_cast<const uint8_t*>(gate->first.biases);
    a.u_codes = static_cast<const uint8_t*>(up->first.codes);
    a.u_scales = static_cast<const uint8_t*>(up->first.scales);
    a.u_biases = static_cast<const uint8_t*>(up->first.biases);
    a.d_codes = static_cast<const uint8_t*>(down->first.codes);
    a.d_scales = static_cast<const uint8_t*>(down->first.scales);
    a.d_biases = static_cast<const uint8_t*>(down->first.biases);
    a.gu_cstride = gate->codes_stride;
    a.gu_sstride = gate->scales_stride;
    a.u_cstride = up->codes_stride;
    a.u_sstride = up->scales_stride;
    a.d_cstride = down->codes_stride;
    a.d_sstride = down->scales_stride;
    a.sg_codes = static_cast<const u32x4*>(sg->codes);
    a.sg_scales = static_cast<const uint16_t*>(sg->scales);
    a.sg_biases = static_cast<const uint16_t*>(sg->biases);
    a.su_codes = static_cast<const u32x4*>(su->codes);
    a.su_scales = static_cast<const uint16_t*>(su->scales);
    a.su_biases = static_cast<const uint16_t*>(su->biases);
    a.sd_codes = static_cast<const u32x4*>(sd->codes);
    a.sd_scales = static_cast<const uint16_t*>(sd->scales);
    a.sd_biases = static_cast<const uint16_t*>(sd->biases);
    a.E = gate->count;
    a.hidden = gate->first.cols;
    a.inter = gate->first.rows;
    a.top_k = top_k;
    a.boundary = boundary;
    float* w = static_cast<float*>(ws);
    a.logits = w;
    a.gate_logit = w + a.E;
    a.act = w + ((a.E + 4) & ~3);        // 16-byte aligned
    a.out = static_cast<_Float16*>(out);
    a.ids = ids;
    a.weights = weights;

    hipError_t e;
    switch (a.hidden / 512) {
        case 1: e = launch_all<1>(a, s); break;
        case 2: e = launch_all<2>(a, s); break;
        case 3: e = launch_all<3>(a, s); break;
        case 4: e = launch_all<4>(a, s); break;
        case 5: e = launch_all<5>(a, s); break;
        case 6: e = launch_all<6>(a, s); break;
        case 7: e = launch_all<7>(a, s); break;
        case 8: e = launch_all<8>(a, s); break;
        default: return dhp_fail(DHP_ERR_UNSUPPORTED, "hidden=%d", a.hidden);
    }
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "moe launch: %s", hipGetErrorString(e));
    return DHP_OK;
}
