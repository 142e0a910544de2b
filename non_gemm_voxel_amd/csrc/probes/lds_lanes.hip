// LDS lane-grouping probe for gfx950: which lanes of a wave the LDS serves in
// one pass, per access type, and the bank rule of 8-byte stores. The lane
// maps in ../lncc_maps.hpp (written by ../gen_lncc_maps.py) rest on what it
// measures. It is a measurement tool, not part of the library.
//
// Build and run (one MI355X; read the counters per dispatch):
//   hipcc -O2 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops lds_lanes.hip -o lds_lanes
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS --kernel-include-regex probe \
//             --output-format csv -d <dir> -o p -- ./lds_lanes
// Part 1 (pair tests, 1 block): only lanes a and b are active, a at byte 0 and
// b at byte 256 (the same banks, other dwords); a conflict count of `iters`
// per dispatch means a and b share a pass. Dispatch order: for each access
// type (8-byte read, 16-byte read, 8-byte write, 16-byte write), for each
// anchor a in {0, 5, 21, 32, 37, 53}, for b = 0..63 (b != a).
// Part 2 (store patterns, 1024 blocks of one wave): every lane writes at the
// byte offset the pattern gives; cycles and conflicts per instruction are
// SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT over SQ_INSTS_LDS. Patterns are
// listed in main() in dispatch order.
// Every address stays inside the 8 KB LDS array (checked on the host).
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>

typedef double d2 __attribute__((ext_vector_type(2)));
constexpr int kLdsDoubles = 1024;

__device__ inline void access(int mode, unsigned base, double &acc, int it) {
    if (mode == 0) {
        double v;
        asm volatile("ds_read_b64 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base));
        acc += v;
    } else if (mode == 1) {
        d2 v;
        asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base));
        acc += v.x + v.y;
    } else if (mode == 2) {
        const double v = double(it);
        asm volatile("ds_write_b64 %0, %1\n s_waitcnt lgkmcnt(0)" : : "v"(base), "v"(v));
    } else {
        const d2 v = {double(it), 1.0};
        asm volatile("ds_write_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : : "v"(base), "v"(v));
    }
}

// Part 1: lanes a and b active.
__global__ __launch_bounds__(64) void probe_pair(int mode, int a, int b, int iters, double *out) {
    __shared__ __align__(16) double lds[kLdsDoubles];
    const int l = threadIdx.x;
    for (int i = l; i < kLdsDoubles; i += 64) lds[i] = i;
    __syncthreads();
    double acc = 0.0;
    if (l == a || l == b) {
        const unsigned base = unsigned(reinterpret_cast<uintptr_t>(lds)) + (l == a ? 0u : 256u);
        for (int it = 0; it < iters; ++it) access(mode, base, acc, it);
    }
    out[l] = acc;
}

// Part 2: every lane at tab[lane] bytes.
__global__ __launch_bounds__(64) void probe_pattern(const unsigned *tab, int mode, int iters, double *out) {
    __shared__ __align__(16) double lds[kLdsDoubles];
    const int l = threadIdx.x;
    for (int i = l; i < kLdsDoubles; i += 64) lds[i] = i;
    __syncthreads();
    double acc = 0.0;
    const unsigned base = unsigned(reinterpret_cast<uintptr_t>(lds)) + tab[l];
    for (int it = 0; it < iters; ++it) access(mode, base, acc, it);
    __syncthreads();
    out[blockIdx.x * 64 + l] = acc + lds[l];
}

int main() {
    struct Pat {
        const char *name;
        int mode;
        unsigned (*f)(int);
    };
    const Pat pats[] = {
        {"w64 16 lanes contiguous 128 B", 2, [](int l) { return 8u * l; }},
        {"w64 contiguous, +64 B", 2, [](int l) { return 8u * l + 64u; }},
        {"w64 contiguous, lanes permuted (l^8)", 2, [](int l) { return 8u * (l ^ 8); }},
        {"w64 contiguous, +32 B", 2, [](int l) { return 8u * l + 32u; }},
        {"w64 16-byte stride (distinct banks)", 2, [](int l) { return 16u * l; }},
        {"w64 two 64 B runs 128 B apart", 2, [](int l) { return 8u * ((l & 7) + 16 * (l >> 3)); }},
        {"w64 816-byte stride", 2, [](int l) { return (816u * (l & 15)) % 4096u + 8u * (l >> 4); }},
        {"w64 32-byte stride", 2, [](int l) { return (32u * l) % 4096u; }},
        {"w128 8 lanes contiguous 128 B", 3, [](int l) { return 16u * l; }},
        {"w128 32-byte stride", 3, [](int l) { return (32u * l) % 4096u; }},
        {"r64 32 lanes contiguous", 0, [](int l) { return 8u * l; }},
        {"r128 16 lanes contiguous", 1, [](int l) { return 16u * l; }},
    };
    const int npat = sizeof(pats) / sizeof(pats[0]);
    for (int i = 0; i < npat; ++i)
        for (int l = 0; l < 64; ++l)
            if (pats[i].f(l) + 16 > 8u * kLdsDoubles) {
                printf("pattern %d out of bounds\n", i);
                return 3;
            }
    double *out;
    unsigned *tab;
    if (hipMalloc(&out, 1024 * 64 * sizeof(double)) != hipSuccess || hipMalloc(&tab, 64 * 4) != hipSuccess) return 1;
    const int anchors[] = {0, 5, 21, 32, 37, 53};
    for (int mode = 0; mode < 4; ++mode)
        for (int a : anchors)
            for (int b = 0; b < 64; ++b)
                if (b != a) hipLaunchKernelGGL(probe_pair, dim3(1), dim3(64), 0, 0, mode, a, b, 2000, out);
    if (hipDeviceSynchronize() != hipSuccess) return 2;
    for (int i = 0; i < npat; ++i) {
        std::vector<unsigned> t(64);
        for (int l = 0; l < 64; ++l) t[l] = pats[i].f(l);
        if (hipMemcpy(tab, t.data(), 64 * 4, hipMemcpyHostToDevice) != hipSuccess) return 1;
        hipLaunchKernelGGL(probe_pattern, dim3(1024), dim3(64), 0, 0, tab, pats[i].mode, 1000, out);
        if (hipDeviceSynchronize() != hipSuccess) return 2;
        printf("pattern %d: %s\n", i, pats[i].name);
    }
    printf("lds_lanes done\n");
    return 0;
}
