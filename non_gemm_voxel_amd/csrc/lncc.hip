// Fused LNCC loss and gradient in one pass with O(1) extra device memory
// ("A Scalable Distributed Framework for Multimodal GigaVoxel Image
// Registration", Key design 2: the moment images, their w-box sums and the
// gradient are all computed on chip).
//
// cc = cross^2 / (v_F v_W + eps) from window sums s_F, s_W, s_FF, s_WW, s_FW;
// with alpha = dcc/ds_FW, beta = dcc/ds_WW, gamma = dcc/ds_W the gradient is
//   gW(y) = -(weight/N) [box(gamma) + 2 W(y) box(beta) + F(y) box(alpha)](y),
// a second box over the coefficient fields. Both boxes have radius R, so an
// output needs inputs 2R away in every direction.
//
// One work item = a TX x TY column tile of the volume and a chunk of output
// planes. A block marches up the chunk one input plane zi at a time. Its
// stages:
//   A  moments on the tile plus a 2R halo: each lane owns NC consecutive
//      columns of one row and keeps their running fp64 z-sums (planes
//      zi-2R..zi) in registers; the plane leaving the window is re-read from
//      global memory (L2). The x-box runs across the 16 lanes of a DPP row
//      (a row of the region fits in one), and the x-boxed sums go to LDS
//      transposed (row index fastest), double-buffered by plane parity.
//   BC one thread per column and pair of rows: the y-box slides down the
//      column, giving the five window sums at plane zc = zi - R, then cc
//      (tile interior -> loss) and alpha, beta, gamma on the tile + R halo.
//   D  x-box of the three coefficient fields along rows, stored transposed.
//   E  one thread per output column: y-box from one contiguous LDS run, then
//      a register ring of the last 2R+1 planes gives the z-box at plane
//      zo = zi - 2R, and the gradient is written there.
// The stages are skewed by a plane so that one barrier interval holds E of
// the previous plane, BC of this one and A of the next (LDS-bound and
// register-only work side by side), and a second holds D: two barriers per
// plane.
// LDS accesses follow how gfx950 serves a wave (64 banks of 4 bytes;
// 16-byte reads 16 lanes per pass in two interleaved lane groups of each
// half-wave, 8-byte reads 32 lanes, 8-byte stores 16 lanes): E reads its run
// with 16-byte loads, BC and D take their tasks from lane maps that keep
// their passes conflict-free (radius 4), and stores stay single 8-byte
// stores. Items are walked in strips of tile rows so that the tiles an XCD
// runs at once share their halos in its L2.
// All window arithmetic is fp64: the variance terms cancel s_FF against
// s_F^2/n and the gradient cancels F box(alpha) against box(gamma); fp32
// sums miss the 1e-3 gradient bar. fp64 adds issue at half the unpacked fp32
// rate on gfx950, but the kernel is bound by latency at two waves per SIMD
// (its fp64 state fills the register file), not by that rate.
#include "lncc_maps.hpp"
#include "mi_device.hpp"
#include "sampler_device.hpp"

namespace ngv {
namespace {

constexpr int kThreads = 512;
constexpr int kTX = 32;
constexpr int kStrip = 8;  // tile rows per strip of the item walk

// LDS row strides in doubles: 2 mod 4, so rows stay 16-byte aligned and
// consecutive rows start on 16-byte bank groups that step by an odd count
// (16 consecutive rows cover all 16 groups of the 64 banks).
constexpr int pad2m4(int n) { return n + ((6 - n % 4) % 4); }

template <int R>
struct Cfg {
    static constexpr int W = 2 * R + 1;
    // the moment region's TY + 4R rows fill at most the 32 DPP rows of a block
    static constexpr int TX = kTX, TY = R <= 4 ? 16 : 32 - 4 * R;
    static constexpr int AX = TX + 4 * R, AY = TY + 4 * R;  // moment region
    static constexpr int CX = TX + 2 * R, CY = TY + 2 * R;  // coefficient region
    static constexpr int NC = (AX + 15) / 16;               // columns per lane in stage A
    static constexpr int ROWP = pad2m4(AY), CXP = pad2m4(CX), TYP = pad2m4(CY);
    static constexpr int L_XB = 5 * CX * ROWP;  // x-boxed z-sums [5][CX][ROWP]
    static constexpr int L_CO = 3 * CY * CXP;   // coefficients [3][CY][CXP]
    static constexpr int L_CT = 3 * TX * TYP;   // x-boxed coefficients [3][TX][TYP]
    static_assert(AY <= kThreads / 16, "one region row per 16 lanes");
    static_assert(NC * 16 >= AX, "a region row fits in one DPP row");
    static_assert(CX * (CY / 2) <= kThreads && CY % 2 == 0, "one BC task per thread");
    static_assert(3 * CY * (TX / 8) <= kThreads, "one D task per thread");
    static_assert(TX * TY <= kThreads, "one output column per thread");
};

// A compiler-only barrier between two LDS stores: it keeps them separate
// 8-byte stores (16 lanes per pass on gfx950) instead of one ds_write2_b64,
// which the hardware serves at half that rate.
__device__ inline void lds_store_fence() { asm volatile("" ::: "memory"); }

// The value v holds in lane (this lane + K) of the same 16-lane DPP row;
// 0 past the row's end.
template <int K>
__device__ inline double from_right(double v) {
    static_assert(K >= 1 && K <= 15, "row shift");
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x100 + K, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x100 + K, 0xF, 0xF, true);
    return __hiloint2double(hi, lo);
}

// Column k of this lane's row neighbourhood: k < NC is its own, beyond that
// lane (k / NC) to the right holds it.
template <int NC, int K>
__device__ inline double col_at(const double (&v)[NC]) {
    if constexpr (K < NC) return v[K];
    else return from_right<K / NC>(v[K % NC]);
}

template <int NC, int R, int J>
__device__ inline void xbox_slide(const double (&v)[NC], double &o, double (&xb)[NC]) {
    if constexpr (J < NC) {
        o += col_at<NC, J + 2 * R>(v) - v[J - 1];
        xb[J] = o;
        xbox_slide<NC, R, J + 1>(v, o, xb);
    }
}

template <int NC, int K, int Q>
__device__ inline void add_block_sums(double t, double &o) {
    if constexpr (K < Q) {
        o += from_right<K>(t);
        add_block_sums<NC, K + 1, Q>(t, o);
    }
}

template <int NC, int I, int REM, int Q>
__device__ inline void add_partial(const double (&v)[NC], double &o) {
    if constexpr (I < REM) {
        o += from_right<Q>(v[I]);
        add_partial<NC, I + 1, REM, Q>(v, o);
    }
}

// x-box across a DPP row: xb[j] = sum of region columns NC*L + j .. NC*L + j + 2R
// (L = lane within the row). Every lane of the wave must call it.
template <int R, int NC>
__device__ inline void xbox_dpp(const double (&v)[NC], double (&xb)[NC]) {
    constexpr int W = 2 * R + 1, Q = W / NC, REM = W % NC;
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < NC; ++j) t += v[j];
    double o = t;
    add_block_sums<NC, 1, Q>(t, o);
    add_partial<NC, 0, REM, Q>(v, o);
    xb[0] = o;
    xbox_slide<NC, R, 1>(v, o, xb);
}

// Sliding box sum along one line: out[o] = sum_{i=0..2R} in[o+i], o < SEG.
template <int R, int SEG>
__device__ inline void slide(const double *in, double (&out)[SEG]) {
    double v[SEG + 2 * R];
#pragma unroll
    for (int i = 0; i < SEG + 2 * R; ++i) v[i] = in[i];
    double s = 0.0;
#pragma unroll
    for (int i = 0; i <= 2 * R; ++i) s += v[i];
#pragma unroll
    for (int o = 0; o < SEG; ++o) {
        out[o] = s;
        if (o + 1 < SEG) s += v[o + 1 + 2 * R] - v[o];
    }
}

// 1/D in fp64: the hardware estimate refined by two Newton steps (each
// doubles the correct bits of the ~2^-26 estimate), for D > 0.
__device__ inline double recip(double d) {
    double r = __builtin_amdgcn_rcp(d);
    r = fma(r, fma(-d, r, 1.0), r);
    r = fma(r, fma(-d, r, 1.0), r);
    return r;
}

struct LnccArgs {
    const float *F;
    const float *W;
    float *gW;
    int64_t nx, ny, nz;
    int64_t tiles_x, tiles_y, chunk, nchunks;
    double eps, gscale;  // gscale = -weight / N
    int accumulate;
    double *partials;
};

// The fused second sweep of a registration step: W is not read but sampled
// from the moving image at every voxel the kernel needs it (the sampler's own
// device functions, so the values are the sampler forward's bit for bit),
// and at each output voxel the LNCC gradient, plus the MI gradient from the
// log-ratio table of the MI forward, feeds the sampler backward there: gu and
// the affine sums are the outputs, W and gW never exist in memory.
struct LnccFuse {
    WarpGeom g;           // the sampler on the output grid (whole moving image)
    int64_t n;            // output voxels (u, gu are 3 volumes of n)
    float *gu;            // sampler backward output
    float sv[9];          // S_v in fp32 (gu = S_v^T g_p)
    int mi;               // add the MI gradient
    MiParams p;           // MI parameters
    const float *table;   // log-ratio table of the MI forward (global memory)
    float mi_gscale;      // mi_grad_scale(p, n)
};

// W at output voxel (x, y, z) (linear index idx) by the sampler.
__device__ inline float sample_w(const LnccFuse &fz, int64_t x, int64_t y, int64_t z, int64_t idx) {
    const float *u = fz.g.u;
    sampler::Sample q;
    sampler::gather(fz.g, int(x), int(y), int(z), u[idx], u[idx + fz.n], u[idx + 2 * fz.n], q);
    return sampler::trilerp(q.c, q.fx, q.fy, q.fz);
}

// Stage-A inputs of plane zi for this lane's NC columns: F, W at zi and at
// the plane leaving the window; zero outside the volume or the region. With
// kF, W is sampled rather than read.
template <int R, bool kF>
__device__ inline void fetch_a(const LnccArgs &a, const LnccFuse &fz, int64_t rowoff, int64_t gx0, int64_t gy,
                               bool row_ok, int64_t zi, int64_t zbeg, float (&v)[Cfg<R>::NC][4]) {
    using C = Cfg<R>;
    const int64_t plane = a.nx * a.ny;
    const int64_t zold = zi - C::W;
    const bool add_new = row_ok && zi >= 0 && zi < a.nz;
    const bool sub_old = row_ok && zold >= zbeg && zold >= 0 && zold < a.nz;
#pragma unroll
    for (int j = 0; j < C::NC; ++j) {
        v[j][0] = v[j][1] = v[j][2] = v[j][3] = 0.0f;
        const int64_t gx = gx0 + j;
        if (gx >= 0 && gx < a.nx) {
            if (add_new) {
                v[j][0] = a.F[zi * plane + rowoff + j];
                if constexpr (kF)
                    v[j][1] = sample_w(fz, gx, gy, zi, zi * plane + rowoff + j);
                else
                    v[j][1] = a.W[zi * plane + rowoff + j];
            }
            if (sub_old) {
                v[j][2] = a.F[zold * plane + rowoff + j];
                if constexpr (kF)
                    v[j][3] = sample_w(fz, gx, gy, zold, zold * plane + rowoff + j);
                else
                    v[j][3] = a.W[zold * plane + rowoff + j];
            }
        }
    }
}

// fn(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile
// time (a plain loop over the ring slots with a data-dependent exit is not
// unrolled for the larger windows, which sends the ring to scratch memory).
template <int B, int E, typename Fn>
__device__ __attribute__((always_inline)) inline void static_for(Fn &&fn) {
    if constexpr (B < E) {
        fn(std::integral_constant<int, B>{});
        static_for<B + 1, E>(fn);
    }
}

// Five window sums -> cc and the coefficient fields.
struct Coef {
    double al, be, ga, cc;
};
__device__ inline Coef coefs(double sF, double sW, double sFF, double sWW, double sFW, double inv_n, double eps) {
    const double cross = sFW - sF * sW * inv_n;
    const double vF = sFF - sF * sF * inv_n;
    const double vW = sWW - sW * sW * inv_n;
    const double invD = recip(vF * vW + eps);
    Coef c;
    c.cc = cross * cross * invD;
    c.al = 2.0 * cross * invD;
    c.be = -c.cc * vF * invD;
    c.ga = -(c.al * sF + 2.0 * c.be * sW) * inv_n;
    return c;
}

// Stage A for one plane: the running z-sums of this lane's NC columns take
// the entering plane and drop the leaving one.
template <int NC>
__device__ inline void a_update(double (&S)[NC][5], const float (&pre)[NC][4]) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const double f = pre[j][0], w = pre[j][1], fo = pre[j][2], wo = pre[j][3];
        // the products of fp32 values are exact in fp64: entering and
        // leaving terms go straight into the sums, one fma each
        S[j][0] += f - fo;
        S[j][1] += w - wo;
        S[j][2] = fma(-fo, fo, fma(f, f, S[j][2]));
        S[j][3] = fma(-wo, wo, fma(w, w, S[j][3]));
        S[j][4] = fma(-fo, wo, fma(f, w, S[j][4]));
    }
}

// Stage A, second half: x-box of the z-sums across the DPP row. Every lane
// of the wave must call it.
template <int R>
__device__ inline void a_xbox(const double (&S)[Cfg<R>::NC][5], double (&o)[5][Cfg<R>::NC]) {
    constexpr int NC = Cfg<R>::NC;
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        double v[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) v[j] = S[j][f];
        xbox_dpp<R, NC>(v, o[f]);
    }
}

// The x-boxed sums stored transposed into xb[5][CX][ROWP].
template <int R>
__device__ inline void a_write(const double (&o)[5][Cfg<R>::NC], double *xb, int ar, int aL) {
    using C = Cfg<R>;
#pragma unroll
    for (int f = 0; f < 5; ++f)
#pragma unroll
        for (int j = 0; j < C::NC; ++j) {
            const int c = C::NC * aL + j;
            if (c < C::CX && (C::AY == kThreads / 16 || ar < C::AY)) xb[(f * C::CX + c) * C::ROWP + ar] = o[f][j];
            lds_store_fence();
        }
}

template <int R>
__device__ inline void a_store(const double (&S)[Cfg<R>::NC][5], double *xb, int ar, int aL) {
    double o[5][Cfg<R>::NC];
    a_xbox<R>(S, o);
    a_write<R>(o, xb, ar, aL);
}

// Stage BC: the y-box down region column bc over rows 2bs .. 2bs + 2R + 1
// gives the window sums at coefficient rows 2bs, 2bs + 1 of plane zc (the two
// boxes share their middle 2R rows); from them cc (tile interior -> loss) and
// the coefficient fields. The loads are 16-byte aligned (ROWP is even).
template <int R>
__device__ inline void bc_load(const double *xb, int bc, int bs, double (&v)[5][2 * R + 2]) {
    using C = Cfg<R>;
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        const double *p = static_cast<const double *>(
            __builtin_assume_aligned(xb + (f * C::CX + bc) * C::ROWP + 2 * bs, 16));
#pragma unroll
        for (int i = 0; i < 2 * R + 2; ++i) v[f][i] = p[i];
    }
}

template <int R>
__device__ inline void bc_compute(const LnccArgs &a, const double (&v)[5][2 * R + 2], double *coef, int bc, int bs,
                                  int64_t x0, int64_t y0, int64_t zc, int64_t zs, int64_t ze, double inv_n,
                                  double &loss_acc) {
    using C = Cfg<R>;
    double ws[5][2];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        double t = v[f][1];
#pragma unroll
        for (int i = 2; i <= 2 * R; ++i) t += v[f][i];
        ws[f][0] = t + v[f][0];
        ws[f][1] = t + v[f][2 * R + 1];
    }
    const int64_t gx = x0 - R + bc;
    const bool xin = gx >= 0 && gx < a.nx && zc >= 0 && zc < a.nz;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int cy = 2 * bs + k;
        const int64_t gy = y0 - R + cy;
        Coef c{0.0, 0.0, 0.0, 0.0};
        if (xin && gy >= 0 && gy < a.ny) {
            c = coefs(ws[0][k], ws[1][k], ws[2][k], ws[3][k], ws[4][k], inv_n, a.eps);
            if (bc >= R && bc < R + C::TX && cy >= R && cy < R + C::TY && zc >= zs && zc < ze) loss_acc += c.cc;
        }
        coef[(0 * C::CY + cy) * C::CXP + bc] = c.al;
        coef[(1 * C::CY + cy) * C::CXP + bc] = c.be;
        coef[(2 * C::CY + cy) * C::CXP + bc] = c.ga;
    }
}

typedef double double2v __attribute__((ext_vector_type(2)));

// Stage E: y-box of the x-boxed coefficients from one aligned LDS run, the
// z-box through the register ring, and the gradient at the output voxel.
// The fused sweep's state at the output voxel: W and dW/dp_vox of its sample
// (from the gathers of the interval before), and the thread's fp64 affine sums.
struct FuseOut {
    float dw[3];
    float ii[3];
    double aff[12];
};

template <int R, bool kF>
__device__ inline void e_stage(const LnccArgs &a, const LnccFuse &fz, const double *cxT, int ex, int ey,
                               double (&ring)[3], double (&zs3)[3], bool emit, int64_t oo, float eF, float eW,
                               float eG, FuseOut &fo) {
    using C = Cfg<R>;
    constexpr int W = C::W;
#pragma unroll
    for (int f = 0; f < 3; ++f) {
        // 16-byte loads: the 2 mod 4 row stride spreads 16 lanes over the 64
        // banks for them, while 8-byte pairs (ds_read2_b64) would put lanes
        // ex and ex + 16 on the same banks
        const double2v *q = reinterpret_cast<const double2v *>(cxT + (f * C::TX + ex) * C::TYP + (ey & ~1));
        double v[W + 1];
#pragma unroll
        for (int i = 0; i <= W / 2; ++i) {
            const double2v t = q[i];
            v[2 * i] = t.x;
            v[2 * i + 1] = t.y;
        }
        double s = v[1];
#pragma unroll
        for (int i = 2; i < W; ++i) s += v[i];
        s += (ey & 1) ? v[W] : v[0];
        zs3[f] += s - ring[f];
        ring[f] = s;
    }
    if (emit) {
        const double g = a.gscale * (zs3[2] + 2.0 * double(eW) * zs3[1] + double(eF) * zs3[0]);
        if constexpr (kF) {
            // the sampler backward of the whole similarity gradient: the LNCC
            // term as stored, then the MI term, as the separate calls add them
            float gt = float(g);
            if (fz.mi) gt = gt + mi::grad_value<3>(eF, eW, fz.p, fz.table, fz.mi_gscale);
            const float gp[3] = {fo.dw[0] * gt, fo.dw[1] * gt, fo.dw[2] * gt};
#pragma unroll
            for (int c = 0; c < 3; ++c) fz.gu[oo + c * fz.n] = sampler::su_component(fz.sv, gp, c);
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                fo.aff[j] += double(gp[j]);
#pragma unroll
                for (int c = 0; c < 3; ++c) fo.aff[3 + 3 * j + c] += double(gp[j]) * double(fo.ii[c]);
            }
        } else {
            a.gW[oo] = float(g) + eG;
        }
    }
}

template <int R, bool kF>
__global__ __launch_bounds__(kThreads) void lncc_kernel(LnccArgs a, LnccFuse fz) {
    using C = Cfg<R>;
    constexpr int NC = C::NC, TX = C::TX, TY = C::TY, W = C::W;
    __shared__ __align__(16) double xbT[2][C::L_XB];
    __shared__ __align__(16) double coef[C::L_CO];
    __shared__ __align__(16) double cxT[C::L_CT];
    __shared__ double red[16];
    const int tid = threadIdx.x;
    const int64_t plane = a.nx * a.ny;
    const double inv_n = 1.0 / (double(W) * W * W);
    double loss_acc = 0.0;
    FuseOut fo;
#pragma unroll
    for (int k = 0; k < 12; ++k) fo.aff[k] = 0.0;

    // stage A: region row ar, columns NC*aL .. NC*aL + NC - 1
    const int ar = tid >> 4, aL = tid & 15;
    // stage BC: region column bc, rows 2*bs, 2*bs + 1 of the coefficient region;
    // stage D: field df, coefficient row dr, output columns 8*dsg .. 8*dsg + 7.
    // For radius 4 the thread -> task maps come from a table that keeps every
    // LDS pass of both stages free of bank conflicts (lncc_maps.hpp); other
    // radii take tasks in plain order.
    bool b_on;
    int bc, bs;
    if constexpr (R == 4) {
        static_assert(C::CX == 40 && C::CY == 24 && C::ROWP == 34 && C::CXP == 42, "map built for this layout");
        const unsigned e = kLnccBcMapR4[tid];
        b_on = e != 0xFFFFu;
        bc = b_on ? int(e & 0xFFu) : 0;
        bs = b_on ? int(e >> 8) : 0;
    } else {
        b_on = tid < C::CX * (C::CY / 2);
        bc = tid % C::CX;
        bs = tid / C::CX;
    }
    bool d_on;
    int dr, dsg, df;
    if constexpr (R == 4) {
        static_assert(C::TYP == 26 && TX == 32, "map built for this layout");
        const unsigned e = kLnccDMapR4[tid];
        d_on = e != 0xFFFFu;
        dr = d_on ? int(e & 0xFFu) : 0;
        dsg = d_on ? int((e >> 8) & 0xFu) : 0;
        df = d_on ? int(e >> 12) : 0;
    } else {
        d_on = tid < 3 * C::CY * (TX / 8);
        dr = tid % C::CY;
        dsg = (tid / C::CY) % (TX / 8);
        df = tid / (C::CY * (TX / 8));
    }
    // stage E: output column (ex, ey); a wave's rows all have one parity
    const int lane = tid & 63, wv = tid >> 6;
    const int ex = lane & 31;
    const int ey = wv + 8 * (lane >> 5);
    const bool e_on = ey < TY;

    const int64_t total = a.tiles_x * a.tiles_y * a.nchunks;
    const ItemRange rng = xcd_items(total);
    for (int64_t it = rng.begin; it < rng.end; it += rng.step) {
        // z-chunk slowest; within a chunk, strips of kStrip tile rows walked
        // column by column, so the ~32 items an XCD runs at once form a compact
        // patch of tiles whose halos and leaving planes stay in its L2 (a walk
        // along whole tile rows kept only the x-halos shared: on the
        // 1280 x 1536 x 1280 grid it fetched 72 B/voxel and took 74 ms, against
        // 60 ms this way)
        const int64_t per_ch = a.tiles_x * a.tiles_y, ch = it / per_ch, r = it - ch * per_ch;
        const int64_t strip = r / (a.tiles_x * kStrip);
        const int64_t h = min(int64_t(kStrip), a.tiles_y - strip * kStrip);
        const int64_t rr = r - strip * a.tiles_x * kStrip;
        const int64_t bx = rr / h, by = strip * kStrip + rr % h;
        const int64_t x0 = bx * TX, y0 = by * TY;
        const int64_t zs = ch * a.chunk;
        const int64_t ze = zs + a.chunk < a.nz ? zs + a.chunk : a.nz;
        const int64_t zbeg = zs - 2 * R, zend = ze + 2 * R;

        const int64_t agy = y0 - 2 * R + ar, agx0 = x0 - 2 * R + NC * aL;
        const bool a_row = ar < C::AY && agy >= 0 && agy < a.ny;
        const int64_t a_off = agy * a.nx + agx0;
        double S[NC][5];
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
            for (int f = 0; f < 5; ++f) S[j][f] = 0.0;
        double ring[W][3];
        double zs3[3] = {0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < W; ++k) ring[k][0] = ring[k][1] = ring[k][2] = 0.0;
        const int64_t gxo = x0 + ex, gyo = y0 + ey;
        // a loss-only call (no gW) has no per-voxel output; the fused sweep
        // always writes gu
        const bool col_in = e_on && gxo < a.nx && gyo < a.ny && (kF || a.gW != nullptr);

        // warm-up: planes zbeg .. zs - 1 only feed the running z-sums
        float pre[NC][4];
        fetch_a<R, kF>(a, fz, a_off, agx0, agy, a_row, zbeg, zbeg, pre);
        for (int64_t zi = zbeg; zi < zs; ++zi) {
            a_update<NC>(S, pre);
            fetch_a<R, kF>(a, fz, a_off, agx0, agy, a_row, zi + 1, zbeg, pre);
        }
        a_update<NC>(S, pre);
        if (zs + 1 < zend) fetch_a<R, kF>(a, fz, a_off, agx0, agy, a_row, zs + 1, zbeg, pre);
        a_store<R>(S, xbT[zs & 1], ar, aL);
        __syncthreads();

        // Per input plane zi >= zs two barrier intervals:
        //   I:  E(zi - 1), BC(zi) from buffer zi & 1, A(zi + 1) into the other buffer
        //   II: D(zi), and the output voxel data for E(zi)
        bool emit = false;
        int64_t oo = 0;
        float eF = 0.0f, eW = 0.0f, eG = 0.0f;
        for (int64_t zb = zs; zb < zend; zb += W) {
            // one input plane; slot is a compile-time constant when unrolled
            auto plane_step = [&](auto sc) __attribute__((always_inline)) {
                const int slot = int(sc);
                const int64_t zi = zb + slot;
                if (zi >= zend) return;  // and so every later slot of this pass
                if (zi > zs) e_stage<R, kF>(a, fz, cxT, ex, ey, ring[(slot + W - 1) % W], zs3, emit, oo, eF, eW, eG, fo);
                if (b_on) {
                    double vb[5][2 * R + 2];
                    bc_load<R>(xbT[zi & 1], bc, bs, vb);
                    bc_compute<R>(a, vb, coef, bc, bs, x0, y0, zi - R, zs, ze, inv_n, loss_acc);
                }
                if (zi + 1 < zend) {
                    a_update<NC>(S, pre);
                    if (zi + 2 < zend) fetch_a<R, kF>(a, fz, a_off, agx0, agy, a_row, zi + 2, zbeg, pre);
                    a_store<R>(S, xbT[(zi + 1) & 1], ar, aL);
                }
                __syncthreads();
                // the output voxel of E(zi) (plane zi - 2R): its F, W and old gW
                const int64_t zo = zi - 2 * R;
                emit = col_in && zo >= zs && zo < ze;
                oo = zo * plane + gyo * a.nx + gxo;
                if (emit) {
                    eF = a.F[oo];
                    if constexpr (kF) {
                        // the output voxel's sample: W and dW/dp_vox for E
                        const float *u = fz.g.u;
                        sampler::Sample q;
                        sampler::gather(fz.g, int(gxo), int(gyo), int(zo), u[oo], u[oo + fz.n], u[oo + 2 * fz.n],
                                        q);
                        sampler::sample_terms(q, eW, fo.dw);
                        fo.ii[0] = float(gxo);
                        fo.ii[1] = float(gyo);
                        fo.ii[2] = float(zo);
                    } else {
                        eW = a.W[oo];
                        if (a.accumulate) eG = a.gW[oo];
                    }
                }
                if (d_on) {
                    double o[8];
                    slide<R, 8>(coef + (df * C::CY + dr) * C::CXP + 8 * dsg, o);
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        cxT[(df * TX + 8 * dsg + k) * C::TYP + dr] = o[k];
                        lds_store_fence();
                    }
                }
                __syncthreads();
                if (zi == zend - 1) e_stage<R, kF>(a, fz, cxT, ex, ey, ring[slot], zs3, emit, oo, eF, eW, eG, fo);
            };
            if constexpr (kF || R > 4) {
                // the fused sweep's sampler state, or radius 5's wider ring,
                // leaves no registers for an unrolled ring: a plain loop (the
                // ring in scratch) spills less and measured faster there
                for (int slot = 0; slot < W; ++slot) plane_step(slot);
            } else {
                // forced unrolling: 3-12% faster than the compiler's own for
                // w = 3..9 on the 640 x 768 x 640 grid (7.37 -> 7.09 ms at w = 9)
                static_for<0, W>(plane_step);
            }
        }
        __syncthreads();
    }
    if constexpr (kF) {
        // slots 0..11: the affine sums (as the sampler backward leaves them),
        // slot 12: the loss
#pragma unroll 1
        for (int k = 0; k < 12; ++k) {
            const double t = block_sum(fo.aff[k], red);
            if (tid == 0) a.partials[size_t(blockIdx.x) * kPartialStride + k] = t;
        }
        const double tot = block_sum(loss_acc, red);
        if (tid == 0) a.partials[size_t(blockIdx.x) * kPartialStride + 12] = tot;
    } else {
        const double tot = block_sum(loss_acc, red);
        if (tid == 0) a.partials[size_t(blockIdx.x) * kPartialStride] = tot;
    }
}

template <int R, bool kF>
hipError_t launch_r(LnccArgs a, const LnccFuse &fz, double weight, double *loss, hipStream_t s, int &nblocks) {
    using C = Cfg<R>;
    a.tiles_x = (a.nx + C::TX - 1) / C::TX;
    a.tiles_y = (a.ny + C::TY - 1) / C::TY;
    // chunk length: a block spends chunk + 2R plane steps on an item plus 2R
    // cheaper warm-up steps, and the busiest CU takes ceil(items / CUs) items;
    // pick the length (1, 2, 4, or a multiple of 8 up to 640) that minimises
    // their product (short chunks only pay on volumes of a few tiles). On the
    // 1280 x 1536 x 1280 grid it picks 640 planes: 55.8-56.1 ms against
    // 56.5 for 320, while a whole-depth chunk (1280, which the product rates
    // lower still) measured 57.8 ms, so longer ones are not offered.
    const int64_t tiles = a.tiles_x * a.tiles_y, cus = device_info().cus;
    int64_t chunk = 8;
    double best = -1.0;
    for (int64_t c = 1; c <= 640; c = c < 8 ? 2 * c : c + 8) {
        const int64_t items = tiles * ((a.nz + c - 1) / c);
        const double cost = double((items + cus - 1) / cus) * (double(c) + 2.8 * R);
        if (best < 0.0 || cost < best) {
            best = cost;
            chunk = c;
        }
        if (c >= a.nz) break;
    }
    a.chunk = chunk;
    a.nchunks = (a.nz + chunk - 1) / chunk;
    const int blocks = persistent_blocks(tiles * a.nchunks, 1);
    nblocks = blocks;
    hipLaunchKernelGGL((lncc_kernel<R, kF>), dim3(blocks), dim3(kThreads), 0, s, a, fz);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const double N = double(a.nx) * double(a.ny) * double(a.nz);
    return launch_partials_final(a.partials + (kF ? 12 : 0), blocks, -weight / N, loss, kF ? 0 : a.accumulate, s);
}

template <bool kF>
hipError_t launch_win(LnccArgs a, const LnccFuse &fz, int win, double weight, double *loss, hipStream_t s,
                      int &nblocks) {
    switch (win / 2) {
        case 1: return launch_r<1, kF>(a, fz, weight, loss, s, nblocks);
        case 2: return launch_r<2, kF>(a, fz, weight, loss, s, nblocks);
        case 3: return launch_r<3, kF>(a, fz, weight, loss, s, nblocks);
        case 4: return launch_r<4, kF>(a, fz, weight, loss, s, nblocks);
        case 5: return launch_r<5, kF>(a, fz, weight, loss, s, nblocks);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_lncc(const float *F, const float *W, int64_t nx, int64_t ny, int64_t nz, int win, float eps,
                       float weight, double *loss, float *gW, int accumulate, void *ws, hipStream_t s) {
    // windows whose tile halo does not fit this kernel's registers and LDS
    if (win > 11) return launch_lncc_big(F, W, nx, ny, nz, win, eps, weight, loss, gW, accumulate, ws, s);
    LnccArgs a;
    a.F = F;
    a.W = W;
    a.gW = gW;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.eps = eps;
    a.gscale = -double(weight) / (double(nx) * double(ny) * double(nz));
    a.accumulate = accumulate;
    a.partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    int nblocks = 0;
    return launch_win<false>(a, LnccFuse{}, win, weight, loss, s, nblocks);
}

hipError_t launch_lncc_fused(const WarpGeom &g, const WarpBwdFinal &fin, const float *F, int win, float eps,
                             float weight, double *loss, const MiFuse *mi, float *gu, double *gA9, double *gt3,
                             int accumulate_affine, void *ws, hipStream_t s) {
    LnccArgs a;
    a.F = F;
    a.W = nullptr;
    a.gW = nullptr;
    a.nx = g.onx;
    a.ny = g.ony;
    a.nz = g.onz;
    a.eps = eps;
    a.gscale = -double(weight) / (double(g.onx) * double(g.ony) * double(g.onz));
    a.accumulate = 0;
    a.partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    LnccFuse fz{};
    fz.g = g;
    fz.n = g.onx * g.ony * g.onz;
    fz.gu = gu;
    for (int k = 0; k < 9; ++k) fz.sv[k] = float(g.sv[k]);
    fz.mi = mi ? 1 : 0;
    if (mi) {
        fz.p = mi->p;
        fz.table = mi->table;
        fz.mi_gscale = mi->gscale;
    }
    int nblocks = 0;
    hipError_t e = launch_win<true>(a, fz, win, weight, loss, s, nblocks);
    if (e != hipSuccess) return e;
    return launch_warp_bwd_final(a.partials, nblocks, fin, gA9, gt3, accumulate_affine, s);
}

}  // namespace ngv
