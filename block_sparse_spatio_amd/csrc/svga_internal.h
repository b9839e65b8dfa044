// Internal helpers of libsvga shared by host code and kernels: division by a
// runtime constant, token geometry, the temporal token order, and each
// executed row's kept key ranges.
//
// Source cited as ASTA: "Accelerating Spatio-Temporal Attention for Video
// Diffusion on TPUs" (Google Developers Blog).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svga.h"

namespace svga {

// Unsigned division of n in [0, 2^31) by a runtime divisor d in [1, 2^31):
// q = (umulhi(n, m) + n) >> s with s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1
// (round-up multiplier; exact for 31-bit n because umulhi(n, m) + n < 2^32).
struct FastDiv {
    uint32_t d, m, s;
    __host__ __device__ FastDiv() : d(1), m(1), s(0) {}
    __host__ explicit FastDiv(uint32_t div) { init(div); }
    __host__ void init(uint32_t div) {
        d = div < 1 ? 1 : div;
        s = 0;
        while ((1ull << s) < d) ++s;
        m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    }
    __host__ __device__ inline uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t hi = __umulhi(n, m);
#else
        uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
        return (hi + n) >> s;
    }
    __host__ __device__ inline void divmod(uint32_t n, uint32_t& q, uint32_t& r) const {
        q = div(n);
        r = n - q * d;
    }
};

// Geometry and mask of one call, with divisors prepared on the host.
struct Geo {
    int32_t F, S, N;       // frames, tokens per frame (H*W), tokens
    int32_t k;             // sink frames
    int32_t bs, bt;        // spatial band (frames), temporal window (flattened positions)
    int32_t layout;        // SVGA_TL_*
    int32_t kS;            // k * S, number of sink tokens
    int32_t Fr;            // F - k, frames after the sink (>= 0)
    FastDiv divS, divF, divFr;
};

__host__ inline Geo make_geo(const svga_geom& g, const svga_mask& m) {
    Geo o;
    o.F = g.F;
    o.S = g.H * g.W;
    o.N = g.F * o.S;
    o.k = m.sink_frames;
    o.bs = m.spatial_band;
    o.bt = m.temporal_band;
    o.layout = m.temporal_layout;
    o.kS = o.k * o.S;
    o.Fr = o.F - o.k;
    o.divS.init((uint32_t)o.S);
    o.divF.init((uint32_t)o.F);
    o.divFr.init((uint32_t)(o.Fr > 0 ? o.Fr : 1));
    return o;
}

// Frame-major token stored at executed position i of a temporal head
// (ASTA Figure 9: (F, H, W) -> (H, W, F)).
__host__ __device__ inline int32_t temporal_src(const Geo& g, int32_t i) {
    uint32_t s, f;
    if (g.layout == SVGA_TL_LITERAL) {
        g.divF.divmod((uint32_t)i, s, f);
    } else {
        if (i < g.kS) return i;
        uint32_t r;
        g.divFr.divmod((uint32_t)(i - g.kS), s, r);
        f = (uint32_t)g.k + r;
    }
    return (int32_t)(f * (uint32_t)g.S + s);
}

// Executed position of frame-major token t in a temporal head.
__host__ __device__ inline int32_t temporal_dst(const Geo& g, int32_t t) {
    uint32_t f, s;
    g.divS.divmod((uint32_t)t, f, s);
    if (g.layout == SVGA_TL_LITERAL) return (int32_t)(s * (uint32_t)g.F + f);
    if ((int32_t)f < g.k) return t;
    return g.kS + (int32_t)s * g.Fr + ((int32_t)f - g.k);
}

// Kept keys of one executed row: up to two disjoint half-open ranges
// [a0, b0) and [a1, b1) with b0 <= a1, plus, for the literal temporal order,
// the sink keys {j : j mod F < k} (`periodic`).
struct RowKeys {
    int32_t a0, b0, a1, b1;
    int32_t periodic;
};

__host__ __device__ inline int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }
__host__ __device__ inline int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }

// ASTA section "Speeding up attention", Figure 3: spatial heads keep the sink
// frames and frames within the band; temporal heads keep the sink frames and
// the spatial window in every frame. Written in executed positions.
__host__ __device__ inline RowKeys row_keys(const Geo& g, int kind, int32_t i) {
    RowKeys r;
    r.periodic = 0;
    if (kind == SVGA_KIND_SPATIAL) {
        int32_t f = (int32_t)g.divS.div((uint32_t)i);
        int32_t lo = imax(0, f - g.bs), hi = imin(g.F - 1, f + g.bs);
        if (lo <= g.k) {  // sink and band touch or overlap: one range
            r.a0 = 0;
            r.b0 = imax(g.k, hi + 1) * g.S;
            r.a1 = r.b1 = r.b0;
        } else {
            r.a0 = 0;
            r.b0 = g.kS;
            r.a1 = lo * g.S;
            r.b1 = (hi + 1) * g.S;
        }
        return r;
    }
    int32_t s;
    if (g.layout == SVGA_TL_LITERAL) {
        s = (int32_t)g.divF.div((uint32_t)i);
        int32_t lo = imax(0, s - g.bt), hi = imin(g.S - 1, s + g.bt);
        r.a0 = r.b0 = 0;
        r.a1 = lo * g.F;
        r.b1 = (hi + 1) * g.F;
        r.periodic = g.k > 0;
        return r;
    }
    if (i < g.kS) {
        uint32_t q, rr;
        g.divS.divmod((uint32_t)i, q, rr);
        s = (int32_t)rr;
    } else {
        s = (int32_t)g.divFr.div((uint32_t)(i - g.kS));
    }
    int32_t lo = imax(0, s - g.bt), hi = imin(g.S - 1, s + g.bt);
    r.a0 = 0;
    r.b0 = g.kS;
    r.a1 = g.kS + lo * g.Fr;
    r.b1 = g.kS + (hi + 1) * g.Fr;
    return r;
}

// Number of sink keys j in [0, x) of the literal order (j mod F < k).
__host__ __device__ inline int32_t periodic_prefix(const Geo& g, int32_t x) {
    uint32_t q, r;
    g.divF.divmod((uint32_t)x, q, r);
    return (int32_t)q * g.k + imin((int32_t)r, g.k);
}

__host__ __device__ inline bool row_keeps(const Geo& g, const RowKeys& r, int32_t j) {
    bool keep = (j >= r.a0 && j < r.b0) || (j >= r.a1 && j < r.b1);
    if (r.periodic && j < g.N) {
        uint32_t q, rr;
        g.divF.divmod((uint32_t)j, q, rr);
        keep = keep || ((int32_t)rr < g.k);
    }
    return keep;
}

// Tile-map byte layout (see svga_tilemap_layout in svga.h).
struct MapLayout {
    int32_t tq, tk;
    size_t n_full, n_bnd, kv, cls, total;
};

__host__ inline MapLayout map_layout(int32_t N, int32_t bq, int32_t bkv) {
    MapLayout L;
    L.tq = (N + bq - 1) / bq;
    L.tk = (N + bkv - 1) / bkv;
    size_t tq = (size_t)L.tq, tk = (size_t)L.tk;
    L.n_full = sizeof(svga_tilemap_header);
    L.n_bnd = L.n_full + 2 * tq * sizeof(int32_t);
    L.kv = L.n_bnd + 2 * tq * sizeof(int32_t);
    L.cls = L.kv + 2 * tq * tk * sizeof(int32_t);
    L.total = (L.cls + 2 * tq * tk + 255) & ~(size_t)255;
    return L;
}

__host__ inline svga_tilemap_header map_header(const svga_geom& g, const svga_mask& m, int32_t bq,
                                               int32_t bkv, int32_t mode, const MapLayout& L) {
    svga_tilemap_header h{};
    h.magic = SVGA_TILEMAP_MAGIC;
    h.version = SVGA_TILEMAP_VERSION;
    h.F = g.F;
    h.H = g.H;
    h.W = g.W;
    h.sink_frames = m.sink_frames;
    h.spatial_band = m.spatial_band;
    h.temporal_band = m.temporal_band;
    h.temporal_layout = m.temporal_layout;
    h.bq = bq;
    h.bkv = bkv;
    h.tq = L.tq;
    h.tk = L.tk;
    h.mode = mode;
    return h;
}

// Class of one tile from its kept-pair count c and valid area a.
__host__ __device__ inline int8_t classify_tile(int mode, int64_t c, int64_t a, bool pad_col) {
    switch (mode) {
        case SVGA_MAP_DENSE:
            return pad_col ? SVGA_TILE_BOUNDARY : SVGA_TILE_FULL;
        case SVGA_MAP_NAIVE:
            return c == 0 ? SVGA_TILE_SKIP : SVGA_TILE_BOUNDARY;
        case SVGA_MAP_EXACT:
            if (c == 0) return SVGA_TILE_SKIP;
            return (c == a && !pad_col) ? SVGA_TILE_FULL : SVGA_TILE_BOUNDARY;
        default: {  // SVGA_MAP_ROUNDED: balanced rounding, majority with ties kept
            bool kept = c > 0 && 2 * c >= a;
            if (!kept) return SVGA_TILE_SKIP;
            return pad_col ? SVGA_TILE_BOUNDARY : SVGA_TILE_FULL;
        }
    }
}

// ---------------------------------------------------------------- kernel launchers (HIP files)

struct AttnLaunch {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const uint8_t* flags;
    const unsigned char* map;
    MapLayout L;
    Geo geo;
    int32_t BH;            // B * n_heads
    int32_t head_dim, bq, bkv, mode, gather;
    float scale;
    int32_t* counter;      // persistent workgroups: work counter in the caller's workspace, or null
    int32_t split;         // 1: the workspace also holds the split-tail region (attn_split_workspace_bytes)
};
hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t stream, bool* supported);
constexpr size_t kAttnWorkspaceBytes = 256;   // the work counter, padded
// Split tail of the persistent launch (kernels of kSplitWaves waves, bq 256
// and 512): at most kSplitItemsMax items, kSplitParts pieces each. Workspace layout: counter at 0; log-sum-exp [items * parts][rows]
// (fp32) at kSplitLseOffset; then the normalised output pieces [items * parts]
// [rows][head_dim] (bf16). rows = the query rows of one workgroup, min(bq, 256).
constexpr int kSplitWaves = 8;
constexpr size_t kSplitItemsMax = 256;
constexpr size_t kSplitParts = 4;
constexpr size_t kSplitLseOffset = 256;
inline size_t split_rows(int32_t bq) { return bq > 256 ? 256 : (size_t)bq; }
inline size_t split_lse_bytes(int32_t bq) { return kSplitItemsMax * kSplitParts * split_rows(bq) * 4; }
inline size_t attn_split_workspace_bytes(int32_t head_dim, int32_t bq) {
    if (bq < 32 * kSplitWaves) return kAttnWorkspaceBytes;   // no split below 256-row workgroups
    return kSplitLseOffset + split_lse_bytes(bq) + kSplitItemsMax * kSplitParts * split_rows(bq) * head_dim * 2;
}
// Tile shapes with a compiled attention kernel (plan_host.cpp).
bool attn_supported(int32_t head_dim, int32_t bq, int32_t bkv);
// Scratch of svga_sparse_attn_fwd_noalloc: the split-tail workspace of the
// largest supported case (head_dim 128, 256-row workgroups), 68,157,696 bytes.
constexpr size_t kNoAllocScratchBytes =
    kSplitLseOffset + kSplitItemsMax * kSplitParts * 256 * 4 + kSplitItemsMax * kSplitParts * 256 * 128 * 2;
// Device address of this device's scratch array (looked up on first use per device).
hipError_t noalloc_scratch(void** out);

hipError_t launch_permute(const void* in, void* out, const uint8_t* flags, int32_t BH, const Geo& g,
                          int32_t head_dim, bool inverse, hipStream_t stream);

hipError_t launch_build_tilemap(const Geo& g, int32_t bq, int32_t bkv, int32_t mode, unsigned char* d_map,
                                const MapLayout& L, const svga_tilemap_header& hdr, hipStream_t stream);

struct RouteLaunch {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* idx;
    int32_t n_samples;
    int32_t BH, head_dim;
    Geo geo;
    float scale;
    void* ws;
    int32_t chunk, n_chunks;
    uint8_t* flags;
    float* err;
};
// Routing runs 64 sample slots per head (slots past n_samples repeat the last sample).
constexpr int kRouteMaxSamples = 64;
// Key chunking and workspace bytes of a routing call (plan_host.cpp).
void route_plan(int32_t BH, int32_t N, int32_t head_dim, int32_t n_samples, int32_t* chunk, int32_t* n_chunks,
                size_t* ws_bytes);
hipError_t launch_route(const RouteLaunch& a, hipStream_t stream);

// Kept pairs of a whole head and the band for a target kept fraction (plan_host.cpp).
int64_t kept_pairs_spatial(int32_t F, int64_t S, int32_t sink, int32_t band);
int64_t kept_pairs_temporal(int32_t F, int64_t S, int32_t sink, int32_t band);
int32_t band_for_kept_fraction(int32_t kind, int32_t F, int64_t S, int32_t sink, double target);

// Host builder (tilemap_host.cpp).
void build_tilemap_host(const Geo& g, int32_t bq, int32_t bkv, int32_t mode, unsigned char* h_map,
                        const MapLayout& L);

}  // namespace svga
