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
// planes. A block marches up the chunk one input plane zi at a time:
//   A  running z-sums (over planes zi-2R..zi) of the five moments on the tile
//      plus a 2R halo, one column per thread slot, fp64 registers; the plane
//      leaving the window is re-read from global memory (L2).
//   B  x-box then y-box in LDS -> the five window sums at plane zc = zi - R
//      on the tile plus an R halo.
//   C  cc (tile interior -> loss) and alpha, beta, gamma on the tile + R halo.
//   D  x-box, y-box of the three coefficient fields in LDS -> tile columns.
//   E  a per-thread register ring of the last 2R+1 planes gives the z-box at
//      plane zo = zi - 2R, and the gradient is written there.
// All window arithmetic is fp64: the variance terms cancel s_FF against
// s_F^2/n and the gradient cancels F box(alpha) against box(gamma); fp32
// sums miss the 1e-3 gradient bar. CDNA's fp64 vector rate equals its plain
// fp32 rate, so this costs registers and LDS bytes, not ALU time.
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kTX = 32, kTY = 16;
constexpr int kThreads = kTX * kTY;  // one thread per output column
constexpr int kSeg = 8;         // outputs per thread in the sliding box passes

constexpr int odd(int v) { return v | 1; }

template <int R>
struct Cfg {
    static constexpr int W = 2 * R + 1;
    static constexpr int AX = kTX + 4 * R, AY = kTY + 4 * R;  // moment region
    static constexpr int CX = kTX + 2 * R, CY = kTY + 2 * R;  // window-sum region
    // LDS row strides, odd in doubles so that lanes walking different rows
    // (x-direction slides) or adjacent columns hit distinct banks
    static constexpr int AXP = odd(AX), CXP = odd(CX), TXP = odd(kTX);
    static constexpr int NA = AX * AY;
    static constexpr int KA = (NA + kThreads - 1) / kThreads;
    static constexpr int LDS_A = 5 * AY * AXP;  // doubles: z-sums; later window sums, x-boxed coefficients
    static constexpr int LDS_B = 5 * AY * CXP;  // doubles: x-boxed z-sums; later coefficients, final boxes
    static_assert(5 * CY * CXP <= LDS_A && 3 * CY * TXP <= LDS_A, "lds_a aliases");
    static_assert(3 * CY * CXP <= LDS_B && 3 * kTY * TXP <= LDS_B, "lds_b aliases");
};

// Sliding box sum along one line: out[o] = sum_{i=0..2R} in[o+i] for the cnt
// (<= kSeg) outputs of one segment.
template <int R, int SEG = kSeg>
__device__ inline void slide(const double *in, int in_stride, double *out, int out_stride, int cnt) {
    double v[SEG + 2 * R];
#pragma unroll
    for (int i = 0; i < SEG + 2 * R; ++i) v[i] = (i < cnt + 2 * R) ? in[i * in_stride] : 0.0;
    double s = 0.0;
#pragma unroll
    for (int i = 0; i <= 2 * R; ++i) s += v[i];
#pragma unroll
    for (int o = 0; o < SEG; ++o) {
        if (o < cnt) out[o * out_stride] = s;
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

// The four values (F, W at the entering plane; F, W at the leaving plane) a
// stage-A slot needs for plane zi; zero where the plane or column is outside.
template <int R>
__device__ inline void fetch_a(const LnccArgs &a, int64_t x0, int64_t y0, int64_t zi, int64_t zbeg, float v[][4]) {
    using C = Cfg<R>;
    const int64_t plane = a.nx * a.ny;
    const int64_t zold = zi - C::W;
    const bool add_new = zi >= 0 && zi < a.nz;
    const bool sub_old = zold >= zbeg && zold >= 0 && zold < a.nz;
#pragma unroll
    for (int k = 0; k < C::KA; ++k) {
        const int q = threadIdx.x + k * kThreads;
        v[k][0] = v[k][1] = v[k][2] = v[k][3] = 0.0f;
        if (q < C::NA) {
            const int ax = q % C::AX, ay = q / C::AX;
            const int64_t gx = x0 - 2 * R + ax, gy = y0 - 2 * R + ay;
            if (gx >= 0 && gx < a.nx && gy >= 0 && gy < a.ny) {
                const int64_t col = gy * a.nx + gx;
                if (add_new) {
                    v[k][0] = a.F[zi * plane + col];
                    v[k][1] = a.W[zi * plane + col];
                }
                if (sub_old) {
                    v[k][2] = a.F[zold * plane + col];
                    v[k][3] = a.W[zold * plane + col];
                }
            }
        }
    }
}

template <int R>
__global__ __launch_bounds__(kThreads) void lncc_kernel(LnccArgs a) {
    using C = Cfg<R>;
    __shared__ double lds_a[C::LDS_A];
    __shared__ double lds_b[C::LDS_B];
    __shared__ double red[16];
    const int tid = threadIdx.x;
    const int tx = tid % kTX, ty = tid / kTX;  // this thread's output column
    const bool owner = true;
    const int64_t plane = a.nx * a.ny;
    const double n = double(C::W) * C::W * C::W, inv_n = 1.0 / n;
    double loss_acc = 0.0;

    const int64_t total = a.tiles_x * a.tiles_y * a.nchunks;
    const ItemRange rng = xcd_items(total);
    for (int64_t it = rng.begin; it < rng.end; it += rng.step) {
        // z-chunk slowest, then y, then x: blocks of one XCD share halo planes
        const int64_t bx = it % a.tiles_x, rest = it / a.tiles_x;
        const int64_t by = rest % a.tiles_y, ch = rest / a.tiles_y;
        const int64_t x0 = bx * kTX, y0 = by * kTY;
        const int64_t zs = ch * a.chunk;
        const int64_t ze = zs + a.chunk < a.nz ? zs + a.chunk : a.nz;

        double S[C::KA][5];
#pragma unroll
        for (int k = 0; k < C::KA; ++k)
#pragma unroll
            for (int f = 0; f < 5; ++f) S[k][f] = 0.0;
        double ring[C::W][3];
        double zs3[3] = {0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < C::W; ++k) ring[k][0] = ring[k][1] = ring[k][2] = 0.0;

        const int64_t zbeg = zs - 2 * R, zend = ze + 2 * R;
        const int64_t gxo = x0 + tx, gyo = y0 + ty;  // this thread's output column
        const bool col_in = owner && gxo < a.nx && gyo < a.ny;
        float pre[C::KA][4];
        fetch_a<R>(a, x0, y0, zbeg, zbeg, pre);

        for (int64_t zb = zbeg; zb < zend; zb += C::W) {
#pragma unroll
            for (int slot = 0; slot < C::W; ++slot) {
                const int64_t zi = zb + slot;
                if (zi >= zend) break;
                // this plane's output voxel (plane zi - 2R): its F, W and old gW
                // are loaded now, used after the last barrier
                const int64_t zo = zi - 2 * R;
                const bool emit = col_in && zo >= zs && zo < ze && a.gW;
                const int64_t oo = zo * plane + gyo * a.nx + gxo;
                float eF = 0.0f, eW = 0.0f, eG = 0.0f;
                if (emit) {
                    eF = a.F[oo];
                    eW = a.W[oo];
                    if (a.accumulate) eG = a.gW[oo];
                }
                // ---- A: running z-sums of the moments on the tile + 2R halo
#pragma unroll
                for (int k = 0; k < C::KA; ++k) {
                    const int q = tid + k * kThreads;
                    if (q < C::NA) {
                        const double f = pre[k][0], w = pre[k][1], fo = pre[k][2], wo = pre[k][3];
                        S[k][0] += f - fo;
                        S[k][1] += w - wo;
                        S[k][2] += f * f - fo * fo;
                        S[k][3] += w * w - wo * wo;
                        S[k][4] += f * w - fo * wo;
                        const int ax = q % C::AX, ay = q / C::AX;
#pragma unroll
                        for (int f5 = 0; f5 < 5; ++f5) lds_a[(f5 * C::AY + ay) * C::AXP + ax] = S[k][f5];
                    }
                }
                // prefetch the next plane's inputs; they arrive during B..E
                if (zi + 1 < zend) fetch_a<R>(a, x0, y0, zi + 1, zbeg, pre);
                __syncthreads();
                if (zi < zs) continue;  // still filling the z-window (uniform)

                // ---- B1: x-box of the z-sums, region A -> (AY rows, CX cols);
                // consecutive lanes take consecutive rows, 4 segments per row
                {
                    constexpr int seg = (C::CX + 3) / 4;
                    for (int w = tid; w < 5 * C::AY * 4; w += kThreads) {
                        const int row = w % C::AY, sg = (w / C::AY) % 4, f = w / (4 * C::AY);
                        const int o0 = sg * seg;
                        const int cnt = C::CX - o0 < seg ? C::CX - o0 : seg;
                        slide<R, seg>(lds_a + (f * C::AY + row) * C::AXP + o0, 1,
                                      lds_b + (f * C::AY + row) * C::CXP + o0, 1, cnt);
                    }
                }
                __syncthreads();
                // ---- B2: y-box -> window sums on (CY, CX), stored over lds_a
                double *wsum = lds_a;  // [5][CY][CXP]
                {
                    constexpr int segs = (C::CY + kSeg - 1) / kSeg;
                    for (int w = tid; w < 5 * C::CX * segs; w += kThreads) {
                        const int col = w % C::CX, sg = (w / C::CX) % segs, f = w / (C::CX * segs);
                        const int o0 = sg * kSeg;
                        const int cnt = C::CY - o0 < kSeg ? C::CY - o0 : kSeg;
                        slide<R>(lds_b + (f * C::AY + o0) * C::CXP + col, C::CXP,
                                 wsum + (f * C::CY + o0) * C::CXP + col, C::CXP, cnt);
                    }
                }
                __syncthreads();
                // ---- C: cc and the coefficient fields at plane zc on (CY, CX)
                const int64_t zc = zi - R;
                double *coef = lds_b;  // [3][CY][CXP]
                for (int q = tid; q < C::CX * C::CY; q += kThreads) {
                    const int cx = q % C::CX, cy = q / C::CX;
                    const int64_t gx = x0 - R + cx, gy = y0 - R + cy;
                    double al = 0.0, be = 0.0, ga = 0.0;
                    if (gx >= 0 && gx < a.nx && gy >= 0 && gy < a.ny && zc >= 0 && zc < a.nz) {
                        const double sF = wsum[(0 * C::CY + cy) * C::CXP + cx];
                        const double sW = wsum[(1 * C::CY + cy) * C::CXP + cx];
                        const double sFF = wsum[(2 * C::CY + cy) * C::CXP + cx];
                        const double sWW = wsum[(3 * C::CY + cy) * C::CXP + cx];
                        const double sFW = wsum[(4 * C::CY + cy) * C::CXP + cx];
                        const double cross = sFW - sF * sW * inv_n;
                        const double vF = sFF - sF * sF * inv_n;
                        const double vW = sWW - sW * sW * inv_n;
                        const double invD = recip(vF * vW + a.eps);
                        const double cc = cross * cross * invD;
                        al = 2.0 * cross * invD;
                        be = -cc * vF * invD;
                        ga = -(al * sF + 2.0 * be * sW) * inv_n;
                        if (cx >= R && cx < R + kTX && cy >= R && cy < R + kTY && zc >= zs && zc < ze) loss_acc += cc;
                    }
                    coef[(0 * C::CY + cy) * C::CXP + cx] = al;
                    coef[(1 * C::CY + cy) * C::CXP + cx] = be;
                    coef[(2 * C::CY + cy) * C::CXP + cx] = ga;
                }
                __syncthreads();
                // ---- D1: x-box of the coefficients -> (CY, TX), over lds_a
                double *cx_box = lds_a;  // [3][CY][TXP]
                {
                    constexpr int segs = kTX / kSeg;
                    for (int w = tid; w < 3 * C::CY * segs; w += kThreads) {
                        const int row = w % C::CY, sg = (w / C::CY) % segs, f = w / (segs * C::CY);
                        const int o0 = sg * kSeg;
                        slide<R>(coef + (f * C::CY + row) * C::CXP + o0, 1, cx_box + (f * C::CY + row) * C::TXP + o0,
                                 1, kSeg);
                    }
                }
                __syncthreads();
                // ---- D2: y-box -> (TY, TX), over lds_b
                double *cxy_box = lds_b;  // [3][TY][TXP]
                {
                    constexpr int segs = kTY / kSeg;
                    for (int w = tid; w < 3 * kTX * segs; w += kThreads) {
                        const int col = w % kTX, sg = (w / kTX) % segs, f = w / (kTX * segs);
                        const int o0 = sg * kSeg;
                        slide<R>(cx_box + (f * C::CY + o0) * C::TXP + col, C::TXP,
                                 cxy_box + (f * kTY + o0) * C::TXP + col, C::TXP, kSeg);
                    }
                }
                __syncthreads();
                // ---- E: z-box through the register ring, gradient at zo
                if (owner) {
#pragma unroll
                    for (int f = 0; f < 3; ++f) {
                        const double v = cxy_box[(f * kTY + ty) * C::TXP + tx];
                        zs3[f] += v - ring[slot][f];
                        ring[slot][f] = v;
                    }
                    if (emit) {
                        const double g = a.gscale * (zs3[2] + 2.0 * double(eW) * zs3[1] + double(eF) * zs3[0]);
                        a.gW[oo] = float(g) + eG;
                    }
                }
                // no barrier needed: the next plane's stage A writes lds_a, last
                // read (as cx_box) before the barrier above; lds_b (read here)
                // is next written after the barrier that ends stage A.
            }
        }
        __syncthreads();
    }
    const double tot = block_sum(loss_acc, red);
    if (tid == 0) a.partials[size_t(blockIdx.x) * kPartialStride] = tot;
}

// One block of 256 threads: thread t sums the partials of blocks t, t+256, ...
// in order, then a fixed-order tree.
__global__ __launch_bounds__(256) void lncc_final(const double *__restrict__ partials, int nblocks, double scale,
                                                  double *__restrict__ loss, int accumulate) {
    __shared__ double red[256];
    const int t = threadIdx.x;
    double s = 0.0;
    for (int b = t; b < nblocks; b += 256) s += partials[size_t(b) * kPartialStride];
    red[t] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) red[t] += red[t + w];
        __syncthreads();
    }
    if (t == 0) {
        const double v = scale * red[0];
        *loss = accumulate ? *loss + v : v;
    }
}

}  // namespace

hipError_t launch_lncc(const float *F, const float *W, int64_t nx, int64_t ny, int64_t nz, int win, float eps,
                       float weight, double *loss, float *gW, int accumulate, void *ws, hipStream_t s) {
    LnccArgs a;
    a.F = F;
    a.W = W;
    a.gW = gW;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.tiles_x = (nx + kTX - 1) / kTX;
    a.tiles_y = (ny + kTY - 1) / kTY;
    // chunk length: long enough to amortise the 4R warm-up planes, short
    // enough to give every CU several items
    const int64_t tiles = a.tiles_x * a.tiles_y;
    int64_t chunk = (nz * tiles + 2 * device_info().cus - 1) / (2 * device_info().cus);
    if (chunk < 8) chunk = 8;
    if (chunk > 128) chunk = 128;
    a.chunk = chunk;
    a.nchunks = (nz + chunk - 1) / chunk;
    a.eps = eps;
    const double N = double(nx) * double(ny) * double(nz);
    a.gscale = -double(weight) / N;
    a.accumulate = accumulate;
    a.partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    const int64_t items = tiles * a.nchunks;
    const int blocks = persistent_blocks(items, 1);
    hipError_t e;
    switch (win / 2) {
        case 1: hipLaunchKernelGGL(lncc_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL(lncc_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 3: hipLaunchKernelGGL(lncc_kernel<3>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL(lncc_kernel<4>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 5: hipLaunchKernelGGL(lncc_kernel<5>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lncc_final, dim3(1), dim3(256), 0, s, a.partials, blocks, -double(weight) / N, loss,
                       accumulate);
    return hipGetLastError();
}

}  // namespace ngv
