// LNCC loss and gradient for large windows, w = 13 .. 31 ("A Scalable
// Distributed Framework for Multimodal GigaVoxel Image Registration", Key
// design 2: moments, window sums, coefficients and the gradient in one
// streaming pass, with extra memory that does not grow with the volume).
//
// The same quantities as the LNCC kernel for small windows: window sums
// s_F, s_W, s_FF, s_WW, s_FW of radius R, cc = cross^2 / (v_F v_W + eps) and
// the coefficient fields alpha, beta, gamma at every voxel of the volume
// (zero outside it), and
//   gW(y) = -(weight/N) [box(gamma) + 2 W(y) box(beta) + F(y) box(alpha)](y).
// The small-window kernel holds a tile's moment region (the tile plus a 2R
// halo) in registers and LDS; at R = 15 that region is 76 x 76 columns for a
// 16 x 16 tile, far beyond a block's registers. Here the running z-sums of
// the five moments over the moment region and, per output column, a ring of
// the last 2R+1 planes of the boxed coefficients live in the block's own
// slice of the workspace (global memory, mostly served by L2 and the
// Infinity Cache; the slice depends on R only, so the workspace is O(1) in
// the volume size), and the per-plane buffers in LDS.
//
// One work item = a 16 x 16 column tile and a chunk of output planes. A
// block marches up the chunk one input plane zi at a time:
//   A   z-sums of the moments on the moment region (the plane leaving the
//       window is read again from F and W); each thread keeps its columns;
//   B   x-box of the z-sums to the coefficient region's columns (in two
//       passes over the columns when their sums do not fit in LDS at once);
//   C   y-box as running sums down the columns -> window sums at plane
//       zc = zi - R, then cc (tile interior -> loss) and the coefficient
//       fields on the tile plus an R halo;
//   D   x-box of the coefficients to the tile's columns;
//   Z   per output column, the y-box of those, the running z-sum through its
//       ring, and the gradient at plane zo = zc - R.
// All window arithmetic is fp64, as in the small-window kernel.
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kBigThreads = 256;
constexpr int kBigT = 16;  // output tile side; one output column per thread
static_assert(kBigT * kBigT == kBigThreads, "stage Z gives each thread one output column");
constexpr size_t kBigLds = 156 * 1024;  // LDS a block may take for the per-plane buffers

__host__ __device__ constexpr size_t round_d(size_t n) { return (n + 31) / 32 * 32; }  // 256-byte multiples

// Sizes for radius R. The per-plane buffers live in LDS: coefficients
// co[3][CX][CX], their x-boxes cxb[3][CX][T], and the x-boxed z-sums
// xb[5][MX][CXH] of CXH coefficient columns at a time -- all CX of them in
// one pass where they fit (R <= 12), else in P = 2 passes.
template <int R>
struct Big {
    static constexpr int W = 2 * R + 1, T = kBigT;
    static constexpr int MX = T + 4 * R;  // moment region side
    static constexpr int CX = T + 2 * R;  // coefficient region side
    static constexpr size_t N_CO = size_t(3) * CX * CX, N_CXB = size_t(3) * CX * T;
    static constexpr int P = (size_t(5) * MX * CX + N_CO + N_CXB) * sizeof(double) <= kBigLds ? 1 : 2;
    static constexpr int CXH = (CX + P - 1) / P;
    static constexpr size_t N_XB = size_t(5) * MX * CXH;
    static constexpr size_t LDS = (N_CO + N_CXB + N_XB) * sizeof(double);
    static_assert(LDS <= kBigLds, "per-plane buffers fit in LDS");
    static constexpr size_t S5 = 0;                                   // z-sums [5][MX][MX]
    static constexpr size_t RING = S5 + round_d(size_t(5) * MX * MX);  // per thread [W][3]
    static constexpr size_t TOTAL = RING + round_d(size_t(W) * 3 * kBigThreads);
};

struct BigArgs {
    const float *F, *W;
    float *gW;
    int64_t nx, ny, nz;
    int64_t tiles_x, tiles_y, chunk, nchunks;
    double eps, gscale;  // gscale = -weight / N
    int accumulate;
    double *partials;
    double *scratch;  // kLnccBigBlocks slices of Big<R>::TOTAL doubles
};

__device__ inline void moments(float f, float w, double (&m)[5]) {
    const double fd = f, wd = w;
    m[0] = fd;
    m[1] = wd;
    m[2] = fd * fd;
    m[3] = wd * wd;
    m[4] = fd * wd;
}

template <int R>
__global__ __launch_bounds__(kBigThreads) void lncc_big_kernel(BigArgs a) {
    using B = Big<R>;
    constexpr int W = B::W, MX = B::MX, CX = B::CX, T = B::T, P = B::P, CXH = B::CXH;
    // C's row segments: about one task per thread over the columns of a pass
    constexpr int S = kBigThreads / CXH < CX ? kBigThreads / CXH : CX, SL = (CX + S - 1) / S;
    const int tid = threadIdx.x;
    double *base = a.scratch + size_t(blockIdx.x) * B::TOTAL;
    double *__restrict__ s5 = base + B::S5;
    double *__restrict__ myring = base + B::RING + size_t(tid) * W * 3;  // this thread's, no other reads it
    extern __shared__ __align__(16) double lds[];
    double *__restrict__ co = lds;
    double *__restrict__ cxb = lds + B::N_CO;
    double *__restrict__ xb = lds + B::N_CO + B::N_CXB;
    const int64_t plane = a.nx * a.ny;
    const double inv_n = 1.0 / (double(W) * W * W);
    const bool grad = a.gW != nullptr;
    __shared__ double red[16];
    double loss_acc = 0.0;

    const int64_t total = a.tiles_x * a.tiles_y * a.nchunks;
    const ItemRange rng = xcd_items(total);
    for (int64_t it = rng.begin; it < rng.end; it += rng.step) {
        const int64_t per_ch = a.tiles_x * a.tiles_y, ch = it / per_ch, r = it - ch * per_ch;
        const int64_t x0 = (r % a.tiles_x) * T, y0 = (r / a.tiles_x) * T;
        const int64_t zs = ch * a.chunk;
        const int64_t ze = zs + a.chunk < a.nz ? zs + a.chunk : a.nz;
        const int64_t zbeg = zs - 2 * R, zend = ze + 2 * R;
        for (int i = tid; i < 5 * MX * MX; i += kBigThreads) s5[i] = 0.0;
        const int tx = tid % T, ty = tid / T;
        const int64_t ox = x0 + tx, oy = y0 + ty;
        double zsum[3] = {0.0, 0.0, 0.0};
        __syncthreads();

        for (int64_t zi = zbeg; zi < zend; ++zi) {
            // A: z-sums over planes zi - 2R .. zi of the moment region columns
            // (each thread keeps its own columns: no barrier needed between planes)
            const int64_t zold = zi - W;
            const bool add_new = zi >= 0 && zi < a.nz;
            const bool sub_old = zold >= zbeg && zold >= 0 && zold < a.nz;
            if (add_new || sub_old) {
                for (int c = tid; c < MX * MX; c += kBigThreads) {
                    const int my = c / MX, mx = c - my * MX;
                    const int64_t gx = x0 - 2 * R + mx, gy = y0 - 2 * R + my;
                    if (gx < 0 || gx >= a.nx || gy < 0 || gy >= a.ny) continue;
                    const int64_t off = gy * a.nx + gx;
                    double mn[5] = {0.0, 0.0, 0.0, 0.0, 0.0}, mo[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
                    if (add_new) moments(a.F[zi * plane + off], a.W[zi * plane + off], mn);
                    if (sub_old) moments(a.F[zold * plane + off], a.W[zold * plane + off], mo);
#pragma unroll
                    for (int f = 0; f < 5; ++f) s5[(f * MX + my) * MX + mx] += mn[f] - mo[f];
                }
            }
            if (zi < zs) continue;  // warm-up: the z-window is not full yet
            __syncthreads();
            const int64_t zc = zi - R;

            // B and C, in P passes over the coefficient columns (P > 1 when
            // the x-boxed sums of all columns do not fit in LDS)
            const bool zc_in = zc >= 0 && zc < a.nz;
            for (int h = 0; h < P; ++h) {
                const int c0 = h * CXH, nc = (c0 + CXH < CX ? c0 + CXH : CX) - c0;
                // B: x-box along each moment-region row to this pass's columns
                for (int t = tid; t < 5 * MX; t += kBigThreads) {
                    const double *src = s5 + size_t(t) * MX + c0;
                    double *dst = xb + size_t(t) * CXH;
                    if constexpr (P == 1 && MX <= 64) {
                        // the row in registers first: its loads all in flight at once
                        double v[MX];
#pragma unroll
                        for (int k = 0; k < MX; ++k) v[k] = src[k];
                        double sum = 0.0;
#pragma unroll
                        for (int k = 0; k < W; ++k) sum += v[k];
                        dst[0] = sum;
#pragma unroll
                        for (int cx = 1; cx < CX; ++cx) {
                            sum += v[cx + W - 1] - v[cx - 1];
                            dst[cx] = sum;
                        }
                    } else {
                        double sum = 0.0;
                        for (int k = 0; k < W; ++k) sum += src[k];
                        dst[0] = sum;
                        for (int j = 1; j < nc; ++j) {
                            sum += src[j + W - 1] - src[j - 1];
                            dst[j] = sum;
                        }
                    }
                }
                __syncthreads();
                // C: down each coefficient column, in S row segments, the five
                // y-boxes as running sums give the window sums at plane zc row
                // by row; from them cc (tile interior -> loss) and the
                // coefficient fields on the tile plus an R halo (zero where
                // the window's centre lies outside the volume)
                for (int t = tid; t < nc * S; t += kBigThreads) {
                    const int j = t % nc, seg = t / nc, cx = c0 + j;
                    const int r0 = seg * SL, r1 = r0 + SL < CX ? r0 + SL : CX;
                    if (r0 >= CX) continue;  // S * SL may overshoot the rows
                    const int64_t gx = x0 - R + cx;
                    const bool col_in = zc_in && gx >= 0 && gx < a.nx;
                    const double *col = xb + j;
                    double ws[5];
#pragma unroll
                    for (int f = 0; f < 5; ++f) {
                        double acc = 0.0;
#pragma unroll
                        for (int k = 0; k < W; ++k) acc += col[(size_t(f) * MX + r0 + k) * CXH];
                        ws[f] = acc;
                    }
                    for (int cy = r0; cy < r1; ++cy) {
                        if (cy > r0) {
#pragma unroll
                            for (int f = 0; f < 5; ++f)
                                ws[f] += col[(size_t(f) * MX + cy + W - 1) * CXH] - col[(size_t(f) * MX + cy - 1) * CXH];
                        }
                        const int64_t gy = y0 - R + cy;
                        double al = 0.0, be = 0.0, ga = 0.0;
                        if (col_in && gy >= 0 && gy < a.ny) {
                            const double sF = ws[0], sW = ws[1], sFF = ws[2], sWW = ws[3], sFW = ws[4];
                            const double cross = sFW - sF * sW * inv_n;
                            const double vF = sFF - sF * sF * inv_n;
                            const double vW = sWW - sW * sW * inv_n;
                            const double invD = 1.0 / (vF * vW + a.eps);
                            const double cc = cross * cross * invD;
                            al = 2.0 * cross * invD;
                            be = -cc * vF * invD;
                            ga = -(al * sF + 2.0 * be * sW) * inv_n;
                            if (cx >= R && cx < R + T && cy >= R && cy < R + T && zc >= zs && zc < ze) loss_acc += cc;
                        }
                        const size_t i = size_t(cy) * CX + cx;
                        co[i] = al;
                        co[size_t(CX) * CX + i] = be;
                        co[size_t(2) * CX * CX + i] = ga;
                    }
                }
                if (h + 1 < P) __syncthreads();  // the next pass overwrites xb
            }
            if (!grad) continue;  // the next plane's stage B starts after a barrier of its own
            __syncthreads();
            // D: x-box of the coefficient rows to the tile's columns
            for (int t = tid; t < 3 * CX; t += kBigThreads) {
                const double *src = co + size_t(t) * CX;
                double *dst = cxb + size_t(t) * T;
                double v[CX];
#pragma unroll
                for (int k = 0; k < CX; ++k) v[k] = src[k];
                double s = 0.0;
#pragma unroll
                for (int k = 0; k < W; ++k) s += v[k];
                dst[0] = s;
#pragma unroll
                for (int x = 1; x < T; ++x) {
                    s += v[x + W - 1] - v[x - 1];
                    dst[x] = s;
                }
            }
            __syncthreads();
            // Z: the y-box at this thread's output column, the z-box through
            // its ring of the last W planes, then the gradient at zo = zc - R
            const int64_t k = zc - (zs - R);  // coefficient planes done before this one
            const int slot = int(k % W);
#pragma unroll
            for (int f = 0; f < 3; ++f) {
                double v = 0.0;
#pragma unroll
                for (int q = 0; q < W; ++q) v += cxb[(size_t(f) * CX + ty + q) * T + tx];
                const double old = k >= W ? myring[slot * 3 + f] : 0.0;
                zsum[f] += v - old;
                myring[slot * 3 + f] = v;
            }
            const int64_t zo = zc - R;
            if (zo >= zs && zo < ze && ox < a.nx && oy < a.ny) {
                const int64_t oo = zo * plane + oy * a.nx + ox;
                const double g = a.gscale * (zsum[2] + 2.0 * double(a.W[oo]) * zsum[1] + double(a.F[oo]) * zsum[0]);
                a.gW[oo] = a.accumulate ? float(g) + a.gW[oo] : float(g);
            }
        }
        __syncthreads();  // the slice is reused by the block's next item
    }
    const double tot = block_sum(loss_acc, red);
    if (tid == 0) a.partials[size_t(blockIdx.x) * kPartialStride] = tot;
}

template <int R>
size_t big_total() {
    return Big<R>::TOTAL;
}

size_t big_total_r(int R) {
    switch (R) {
        case 6: return big_total<6>();
        case 7: return big_total<7>();
        case 8: return big_total<8>();
        case 9: return big_total<9>();
        case 10: return big_total<10>();
        case 11: return big_total<11>();
        case 12: return big_total<12>();
        case 13: return big_total<13>();
        case 14: return big_total<14>();
        case 15: return big_total<15>();
        default: return 0;
    }
}

template <int R>
hipError_t launch_big_r(const BigArgs &a, int blocks, hipStream_t s) {
    using B = Big<R>;
    const size_t lds = B::LDS;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(lncc_big_kernel<R>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(lncc_big_kernel<R>, dim3(blocks), dim3(kBigThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

size_t lncc_big_bytes(int win) {
    if (win < 13 || win > 31) return 0;
    return size_t(kLnccBigBlocks) * big_total_r(win / 2) * sizeof(double);
}

hipError_t launch_lncc_big(const float *F, const float *W, int64_t nx, int64_t ny, int64_t nz, int win, float eps,
                           float weight, double *loss, float *gW, int accumulate, void *ws, hipStream_t s) {
    BigArgs a;
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
    a.scratch = reinterpret_cast<double *>(static_cast<char *>(ws) + lncc_big_offset());
    const int R = win / 2;
    a.tiles_x = (nx + kBigT - 1) / kBigT;
    a.tiles_y = (ny + kBigT - 1) / kBigT;
    // chunk length: an item costs chunk + 4R plane steps (2R warm-up planes
    // of the z-sums, 2R more before its first output) and the busiest block
    // takes ceil(items / blocks) items; pick the length that minimises the
    // product
    const int64_t tiles = a.tiles_x * a.tiles_y;
    int64_t chunk = nz;
    double best = -1.0;
    for (int64_t c = 8; c < nz + 8; c += 8) {
        const int64_t cl = c < nz ? c : nz;
        const int64_t items = tiles * ((nz + cl - 1) / cl);
        const int64_t nb = items < kLnccBigBlocks ? items : kLnccBigBlocks;
        const double cost = double((items + nb - 1) / nb) * (double(cl) + 4.0 * R);
        if (best < 0.0 || cost < best) {
            best = cost;
            chunk = cl;
        }
    }
    a.chunk = chunk;
    a.nchunks = (nz + chunk - 1) / chunk;
    const int64_t items = tiles * a.nchunks;
    int blocks = int(items < kLnccBigBlocks ? items : kLnccBigBlocks);
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;  // whole XCD groups; the walk gives extra blocks no items
    if (blocks > kLnccBigBlocks) blocks = kLnccBigBlocks;
    hipError_t e;
    switch (R) {
        case 6: e = launch_big_r<6>(a, blocks, s); break;
        case 7: e = launch_big_r<7>(a, blocks, s); break;
        case 8: e = launch_big_r<8>(a, blocks, s); break;
        case 9: e = launch_big_r<9>(a, blocks, s); break;
        case 10: e = launch_big_r<10>(a, blocks, s); break;
        case 11: e = launch_big_r<11>(a, blocks, s); break;
        case 12: e = launch_big_r<12>(a, blocks, s); break;
        case 13: e = launch_big_r<13>(a, blocks, s); break;
        case 14: e = launch_big_r<14>(a, blocks, s); break;
        case 15: e = launch_big_r<15>(a, blocks, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const double N = double(nx) * double(ny) * double(nz);
    return launch_partials_final(a.partials, blocks, -double(weight) / N, loss, accumulate, s);
}

}  // namespace ngv
