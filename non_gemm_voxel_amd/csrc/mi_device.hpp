// Device helpers of the Parzen joint histogram and its gradient, shared by
// the MI kernels and the sampler forward that builds the histogram in the
// same sweep ("A Scalable Distributed Framework for Multimodal GigaVoxel
// Image Registration", Key design 2).
#pragma once

#include "ngv_internal.hpp"

namespace ngv {
namespace mi {

constexpr float kFix = 4294967296.0f;  // 2^32: fixed-point scale of the histogram

// Cubic B-spline weights of the four bins ia..ia+3 around bin coordinate c
// (ia = floor(c) - 1, t = c - floor(c)), the uniform cubic B-spline basis.
__device__ inline void bspline4(float c, int &ia, float w[4]) {
    const float fl = floorf(c);
    const float t = c - fl, t2 = t * t, t3 = t2 * t, s = 1.0f - t;
    ia = int(fl) - 1;
    w[0] = s * s * s * (1.0f / 6.0f);
    w[1] = fmaf(3.0f, t3, fmaf(-6.0f, t2, 4.0f)) * (1.0f / 6.0f);
    w[2] = fmaf(-3.0f, t3, fmaf(3.0f, t2, fmaf(3.0f, t, 1.0f))) * (1.0f / 6.0f);
    w[3] = t3 * (1.0f / 6.0f);
}

// Derivatives beta'(b - c) of the same four weights with respect to their
// argument b - c (so d/dc of weight b is minus this).
__device__ inline void bspline4_deriv(float c, int &ia, float d[4]) {
    const float fl = floorf(c);
    const float t = c - fl, t2 = t * t, s = 1.0f - t;
    ia = int(fl) - 1;
    d[0] = 0.5f * s * s;
    d[1] = fmaf(-1.5f, t2, 2.0f * t);
    d[2] = fmaf(1.5f, t2, -0.5f - t);
    d[3] = -0.5f * t2;
}

__device__ inline float bin_coord(float v, float lo, float hi, float scale) {
    return fmaf(fminf(fmaxf(v, lo), hi) - lo, scale, 2.0f);
}

// The fixed image's bin under the zero-order (box) kernel of Mattes et al.'s
// original pair: the integer a with a - c in (-1/2, 1/2], i.e. floor(c + 1/2)
// (a sample half way between two bin centres goes to the upper one), taken on
// the fp32 bin coordinate.
__device__ inline int box_bin(float v, float lo, float hi, float scale) {
    return int(floorf(bin_coord(v, lo, hi, scale) + 0.5f));
}

// The fixed sample's bins: FO = 3, the 4 cubic B-spline weights from bin ia;
// FO = 0, the box bin ia with weight 1 (wa[1..3] = 0, rows never touched).
template <int FO>
__device__ inline void fixed_weights(float fv, const MiParams &p, int &ia, float wa[4]) {
    if constexpr (FO == 0) {
        ia = box_bin(fv, p.f_lo, p.f_hi, p.f_scale);
        wa[0] = 1.0f;
        wa[1] = wa[2] = wa[3] = 0.0f;
    } else {
        bspline4(bin_coord(fv, p.f_lo, p.f_hi, p.f_scale), ia, wa);
    }
}

// d loss / d W at one voxel from the log-ratio table L (bins x bins, in
// LDS): the fixed sample's weights times the derivatives of the moving
// sample's weights, against L, times gscale = weight * (W's bin scale) / N;
// zero where W is clamped. The MI gradient sweep and the sampler backward
// that forms the MI gradient itself share it, so both give the same value.
template <int FO>
__device__ inline float grad_value(float fv, float wv, const MiParams &p, const float *L, float gscale) {
    float g = 0.0f;
    if (wv >= p.w_lo && wv <= p.w_hi) {
        constexpr int kRows = FO == 0 ? 1 : 4;  // fixed bins with weight
        int ia, ib;
        float wa[4], db[4];
        fixed_weights<FO>(fv, p, ia, wa);
        bspline4_deriv(bin_coord(wv, p.w_lo, p.w_hi, p.w_scale), ib, db);
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const float *row = L + (ia + i) * p.bins + ib;
            const float s = fmaf(row[0], db[0], fmaf(row[1], db[1], fmaf(row[2], db[2], row[3] * db[3])));
            g = fmaf(wa[i], s, g);
        }
        g *= gscale;
    }
    return g;
}

// Each thread adds its samples' 4 x 4 weight blocks (1 x 4 with the box
// kernel on the fixed image) into a private 6 x 6 window of the histogram
// held in registers (fp32), anchored one bin below its first sample's block.
// A sample whose block falls outside the window is deferred: the wave
// appends it to its ring of deferred samples in LDS, and once 64 are queued
// all 64 lanes add one each straight to the block's LDS histogram (u64
// atomics of the 32.32 fixed-point products). Deferring keeps the wave
// converged: with noisy intensities a few lanes leave their window at almost
// every step, and adding their blocks at once would run the 16-atomic path
// for the whole wave each time. hist_flush drains the ring and empties the
// window into LDS in 32.32 fixed point -- summed across the wave first when
// every lane shares one anchor (the background, where thousands of samples
// hit the same bins and per-sample atomics would serialise). The fp32 sums
// of a window (at most 64 samples per lane, and a wave's 64 lanes when they
// share an anchor) are the only rounding before the fixed-point sums, which
// are exact and do not depend on order; which way a sample goes depends only
// on the data, so the histogram is the same on every run.
constexpr int kWin = 6;
constexpr int kQueue = 128;  // deferred samples per wave (a power of two, >= 2 x 64)
struct HistCtx {
    float acc[kWin][kWin];
    int ha, hb;
    bool anchored;
    float2 *q;   // this wave's ring of deferred (F, W) samples in LDS
    int qh, qn;  // ring head and count: the same in every lane of the wave
};

// LDS bytes of the deferred-sample rings of a block of `threads` threads.
constexpr size_t ring_bytes(int threads) { return size_t(threads / 64) * kQueue * sizeof(float2); }

// rings: ring_bytes(blockDim.x) of LDS for the block.
__device__ inline void hist_init(HistCtx &c, float2 *rings) {
#pragma unroll
    for (int i = 0; i < kWin; ++i)
#pragma unroll
        for (int j = 0; j < kWin; ++j) c.acc[i][j] = 0.0f;
    c.anchored = false;
    c.ha = c.hb = 0;
    c.q = rings + (threadIdx.x >> 6) * kQueue;
    c.qh = c.qn = 0;
}

__device__ inline void shift6(const float w[4], int d, float e[kWin]) {
    // e[j] = w[j - d] for 0 <= j - d < 4, else 0; d in {0, 1, 2}
    e[0] = d == 0 ? w[0] : 0.0f;
    e[1] = d == 0 ? w[1] : (d == 1 ? w[0] : 0.0f);
    e[2] = d == 0 ? w[2] : (d == 1 ? w[1] : w[0]);
    e[3] = d == 0 ? w[3] : (d == 1 ? w[2] : w[1]);
    e[4] = d == 0 ? 0.0f : (d == 1 ? w[3] : w[2]);
    e[5] = d == 2 ? w[3] : 0.0f;
}

// The n oldest deferred samples of the wave (n <= 64), one per lane, added
// to the LDS histogram. Every lane of the wave must call it.
template <int FO>
__device__ inline void hist_drain(HistCtx &c, int n, const MiParams &p, unsigned long long *h) {
    constexpr int kRows = FO == 0 ? 1 : 4;
    __builtin_amdgcn_wave_barrier();
    const int lane = threadIdx.x & 63, nb = p.bins;
    if (lane < n) {
        const float2 e = c.q[(c.qh + lane) & (kQueue - 1)];
        int ia, ib;
        float wa[4], wb[4];
        fixed_weights<FO>(e.x, p, ia, wa);
        bspline4(bin_coord(e.y, p.w_lo, p.w_hi, p.w_scale), ib, wb);
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const float wi = wa[i] * kFix;
            unsigned long long *row = h + (ia + i) * nb + ib;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned long long q = __float2ull_rn(wi * wb[j]);
                if (q) atomicAdd(row + j, q);
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    c.qh = (c.qh + n) & (kQueue - 1);
    c.qn -= n;
}

// FO: the Parzen kernel of the fixed image (3: cubic B-spline, a 4 x 4 block
// per sample; 0: the box, a 1 x 4 block). valid = false: no sample in this
// lane. Every lane of the wave must call it.
template <int FO = 3>
__device__ inline void hist_add(HistCtx &c, float fv, float wv, bool valid, const MiParams &p,
                                unsigned long long *h) {
    constexpr int kRows = FO == 0 ? 1 : 4;  // fixed bins one sample touches
    bool defer = false;
    if (valid) {
        const int nb = p.bins;
        int ia, ib;
        float wa[4], wb[4];
        fixed_weights<FO>(fv, p, ia, wa);
        bspline4(bin_coord(wv, p.w_lo, p.w_hi, p.w_scale), ib, wb);
        if (!c.anchored) {
            c.ha = min(max(ia - 1, 0), nb - kWin);
            c.hb = min(max(ib - 1, 0), nb - kWin);
            c.anchored = true;
        }
        const int da = ia - c.ha, db = ib - c.hb;
        if (da >= 0 && da <= kWin - kRows && db >= 0 && db <= kWin - 4) {
            float ea[kWin], eb[kWin];
            if constexpr (FO == 0) {
#pragma unroll
                for (int i = 0; i < kWin; ++i) ea[i] = i == da ? 1.0f : 0.0f;
            } else {
                shift6(wa, da, ea);
            }
            shift6(wb, db, eb);
#pragma unroll
            for (int i = 0; i < kWin; ++i)
#pragma unroll
                for (int j = 0; j < kWin; ++j) c.acc[i][j] = fmaf(ea[i], eb[j], c.acc[i][j]);
        } else {
            defer = true;
        }
    }
    const unsigned long long m = __ballot(defer);
    if (m) {
        if (defer) {
            const int lane = threadIdx.x & 63;
            const int rank = __popcll(m & ((1ull << lane) - 1ull));
            c.q[(c.qh + c.qn + rank) & (kQueue - 1)] = make_float2(fv, wv);
        }
        c.qn += __popcll(m);
        if (c.qn >= 64) hist_drain<FO>(c, 64, p, h);
    }
}

// Every lane of the wave must call it.
template <int FO = 3>
__device__ inline void hist_flush(HistCtx &c, const MiParams &p, unsigned long long *h) {
    const int nb = p.bins;
    if (c.qn > 0) hist_drain<FO>(c, c.qn, p, h);
    // lanes without samples carry zeros: give them the first anchored lane's anchor
    const unsigned long long have = __ballot(c.anchored);
    if (have == 0ull) return;
    const int src = __ffsll((long long)have) - 1;
    const int ha0 = __shfl(c.ha, src, 64), hb0 = __shfl(c.hb, src, 64);
    if (!c.anchored) {
        c.ha = ha0;
        c.hb = hb0;
    }
    const bool same = __all(c.ha == ha0 && c.hb == hb0);
    const int lane = threadIdx.x & 63;
    if (same) {
#pragma unroll
        for (int i = 0; i < kWin; ++i)
#pragma unroll
            for (int j = 0; j < kWin; ++j) {
                const float v = wave_sum(c.acc[i][j]);
                if (lane == i * kWin + j) {
                    const unsigned long long q = __float2ull_rn(v * kFix);
                    if (q) atomicAdd(h + (ha0 + i) * nb + hb0 + j, q);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < kWin; ++i)
#pragma unroll
            for (int j = 0; j < kWin; ++j) {
                const unsigned long long q = __float2ull_rn(c.acc[i][j] * kFix);
                if (q) atomicAdd(h + (c.ha + i) * nb + c.hb + j, q);
            }
    }
#pragma unroll
    for (int i = 0; i < kWin; ++i)
#pragma unroll
        for (int j = 0; j < kWin; ++j) c.acc[i][j] = 0.0f;
    c.anchored = false;
}

}  // namespace mi
}  // namespace ngv
