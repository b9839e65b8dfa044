// Device tile-map builder: one workgroup per (query tile, head kind).
//
// Same counting as the host builder (per-row kept key ranges: exact overlap
// for the key tiles at a range's ends, a difference array over key tiles for
// those fully inside), with LDS atomics, then block-wide scans to classify and
// to compact the canonical lists (full tiles ascending, then boundary tiles
// ascending). The result is bit-identical to the host builder's.
// ASTA sections "Logical sparsity is not physical sparsity" (tile classes) and
// "Align the sparse mask with final execution" (balanced rounding).
#include "svga_internal.h"

namespace svga {

namespace {

constexpr int kThreads = 256;

// Exclusive scan of a[0..n) in place (LDS), returns the total. `tmp` holds kThreads ints.
__device__ int32_t block_exclusive_scan(int32_t* a, int32_t n, int32_t* tmp) {
    const int t = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = imin(n, t * per), hi = imin(n, lo + per);
    int32_t s = 0;
    for (int i = lo; i < hi; ++i) s += a[i];
    tmp[t] = s;
    __syncthreads();
    if (t == 0) {
        int32_t run = 0;
        for (int i = 0; i < kThreads; ++i) {
            int32_t x = tmp[i];
            tmp[i] = run;
            run += x;
        }
        tmp[kThreads] = run;
    }
    __syncthreads();
    int32_t run = tmp[t];
    for (int i = lo; i < hi; ++i) {
        int32_t x = a[i];
        a[i] = run;
        run += x;
    }
    const int32_t total = tmp[kThreads];
    __syncthreads();
    return total;
}

__device__ inline void add_range(const Geo& g, int32_t bkv, bool periodic, int32_t a, int32_t b, int32_t* cnt,
                                 int32_t* diff) {
    if (a >= b) return;
    const int32_t ja = a / bkv, jb = (b - 1) / bkv;
    auto psub = [&](int32_t x, int32_t y) { return periodic ? periodic_prefix(g, y) - periodic_prefix(g, x) : 0; };
    if (ja == jb) {
        atomicAdd(&cnt[ja], (b - a) - psub(a, b));
        return;
    }
    const int32_t ea = (ja + 1) * bkv, sb = jb * bkv;
    atomicAdd(&cnt[ja], (ea - a) - psub(a, ea));
    atomicAdd(&cnt[jb], (b - sb) - psub(sb, b));
    if (jb > ja + 1) {
        atomicAdd(&diff[ja + 1], 1);
        atomicAdd(&diff[jb], -1);
    }
}

__global__ __launch_bounds__(kThreads) void tilemap_kernel(Geo g, int32_t bq, int32_t bkv, int32_t mode,
                                                           unsigned char* __restrict__ map, MapLayout L,
                                                           svga_tilemap_header hdr) {
    extern __shared__ int32_t sm[];
    const int32_t tq = L.tq, tk = L.tk, N = g.N;
    int32_t* cnt = sm;                // [tk]
    int32_t* diff = sm + tk;          // [tk + 1]
    int32_t* tmp = sm + 2 * tk + 1;   // [kThreads + 1]
    const int kind = blockIdx.y;
    const int32_t I = blockIdx.x;
    const int t = threadIdx.x;
    if (I == 0 && kind == 0) {
        if (t == 0) *reinterpret_cast<svga_tilemap_header*>(map) = hdr;
        // alignment padding after the class matrix: zero, as the host builder leaves it
        for (size_t p = L.cls + 2 * (size_t)tq * tk + t; p < L.total; p += kThreads) map[p] = 0;
    }

    const bool periodic = kind == SVGA_KIND_TEMPORAL && g.layout == SVGA_TL_LITERAL && g.k > 0;
    const int32_t r0 = I * bq, r1 = imin(N, r0 + bq), rows = r1 - r0;
    for (int32_t j = t; j < tk; j += kThreads) cnt[j] = 0;
    for (int32_t j = t; j <= tk; j += kThreads) diff[j] = 0;
    __syncthreads();
    if (mode != SVGA_MAP_DENSE) {
        for (int32_t i = r0 + t; i < r1; i += kThreads) {
            RowKeys rk = row_keys(g, kind, i);
            add_range(g, bkv, periodic, rk.a0, rk.b0, cnt, diff);
            add_range(g, bkv, periodic, rk.a1, rk.b1, cnt, diff);
        }
    }
    __syncthreads();
    // inclusive prefix of diff = rows whose range covers key tile J entirely
    block_exclusive_scan(diff, tk + 1, tmp);   // diff[J] now holds the sum of diff[0..J)
    int8_t* cls = reinterpret_cast<int8_t*>(map + L.cls) + ((size_t)kind * tq + I) * tk;
    for (int32_t J = t; J < tk; J += kThreads) {
        const int32_t c0 = J * bkv, c1 = imin(N, c0 + bkv), cols = c1 - c0;
        const int64_t area = (int64_t)rows * cols;
        int64_t c = area;
        if (mode != SVGA_MAP_DENSE) {
            const int32_t full_rows = diff[J + 1];
            const int32_t sp = periodic ? periodic_prefix(g, c1) - periodic_prefix(g, c0) : 0;
            c = (int64_t)cnt[J] + (int64_t)full_rows * (cols - sp) + (int64_t)rows * sp;
        }
        const bool pad_col = (int64_t)(J + 1) * bkv > N;
        const int8_t k = classify_tile(mode, c, area, pad_col);
        cls[J] = k;
        cnt[J] = k;   // keep the class for the compaction below
    }
    __syncthreads();
    // flags -> positions: diff[J] = is_full, then diff reused for is_boundary
    for (int32_t J = t; J < tk; J += kThreads) diff[J] = cnt[J] == SVGA_TILE_FULL;
    __syncthreads();
    const int32_t nf = block_exclusive_scan(diff, tk, tmp);
    int32_t* kv = reinterpret_cast<int32_t*>(map + L.kv) + ((size_t)kind * tq + I) * tk;
    for (int32_t J = t; J < tk; J += kThreads)
        if (cnt[J] == SVGA_TILE_FULL) kv[diff[J]] = J;
    __syncthreads();
    for (int32_t J = t; J < tk; J += kThreads) diff[J] = cnt[J] == SVGA_TILE_BOUNDARY;
    __syncthreads();
    const int32_t nb = block_exclusive_scan(diff, tk, tmp);
    for (int32_t J = t; J < tk; J += kThreads)
        if (cnt[J] == SVGA_TILE_BOUNDARY) kv[nf + diff[J]] = J;
    for (int32_t p = nf + nb + t; p < tk; p += kThreads) kv[p] = -1;
    if (t == 0) {
        reinterpret_cast<int32_t*>(map + L.n_full)[(size_t)kind * tq + I] = nf;
        reinterpret_cast<int32_t*>(map + L.n_bnd)[(size_t)kind * tq + I] = nb;
    }
}

}  // namespace

hipError_t launch_build_tilemap(const Geo& g, int32_t bq, int32_t bkv, int32_t mode, unsigned char* d_map,
                                const MapLayout& L, const svga_tilemap_header& hdr, hipStream_t stream) {
    const size_t lds = (size_t)(2 * L.tk + 1 + kThreads + 1) * sizeof(int32_t);
    dim3 grid((unsigned)L.tq, 2);
    hipLaunchKernelGGL(tilemap_kernel, grid, dim3(kThreads), lds, stream, g, bq, bkv, mode, d_map, L, hdr);
    return hipGetLastError();
}

}  // namespace svga
