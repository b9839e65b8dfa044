// C ABI of libsvga: argument checks on the host, then kernel launches.
// Nothing is launched when a check fails.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "svga_internal.h"

using namespace svga;

namespace {

thread_local std::string g_last_error;

svga_status fail(svga_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

svga_status ok() {
    g_last_error.clear();
    return SVGA_OK;
}

svga_status check_geom(const svga_geom* g) {
    if (!g) return fail(SVGA_EINVAL, "geom is NULL");
    if (g->F < 1 || g->H < 1 || g->W < 1) return fail(SVGA_EINVAL, "F, H, W must be >= 1 (got %d, %d, %d)", g->F, g->H, g->W);
    int64_t n = (int64_t)g->F * g->H * g->W;
    if (n >= (int64_t(1) << 30)) return fail(SVGA_EINVAL, "N = F*H*W = %lld must be below 2^30", (long long)n);
    return SVGA_OK;
}

svga_status check_mask(const svga_mask* m, const svga_geom* g) {
    if (!m) return fail(SVGA_EINVAL, "mask is NULL");
    if (m->sink_frames < 0 || m->sink_frames > g->F)
        return fail(SVGA_EINVAL, "sink_frames must be in [0, F=%d] (got %d)", g->F, m->sink_frames);
    if (m->spatial_band < 0 || m->temporal_band < 0) return fail(SVGA_EINVAL, "bands must be >= 0");
    if (m->temporal_layout != SVGA_TL_SINK_FIRST && m->temporal_layout != SVGA_TL_LITERAL)
        return fail(SVGA_EINVAL, "unknown temporal_layout %d", m->temporal_layout);
    return SVGA_OK;
}

svga_status check_tiles(const svga_geom* g, int32_t bq, int32_t bkv) {
    if (bq < 1 || bq > 4096 || bkv < 1 || bkv > 4096)
        return fail(SVGA_EINVAL, "tile sizes must be in [1, 4096] (got bq=%d, bkv=%d)", bq, bkv);
    int64_t n = (int64_t)g->F * g->H * g->W;
    int64_t tq = (n + bq - 1) / bq, tk = (n + bkv - 1) / bkv;
    if (tq * tk >= (int64_t(1) << 28)) return fail(SVGA_EINVAL, "tq*tk = %lld must be below 2^28", (long long)(tq * tk));
    return SVGA_OK;
}

svga_status check_mode(int32_t mode) {
    if (mode < SVGA_MAP_DENSE || mode > SVGA_MAP_ROUNDED) return fail(SVGA_EINVAL, "unknown mode %d", mode);
    return SVGA_OK;
}

svga_status check_heads(int32_t B, int32_t n_heads) {
    if (B < 1 || n_heads < 1) return fail(SVGA_EINVAL, "B and n_heads must be >= 1");
    if ((int64_t)B * n_heads > 65535) return fail(SVGA_EINVAL, "B*n_heads must be at most 65535");
    return SVGA_OK;
}

svga_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SVGA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define TRY(x)                       \
    do {                             \
        svga_status _s = (x);        \
        if (_s != SVGA_OK) return _s; \
    } while (0)

}  // namespace

extern "C" {

const char* svga_status_string(svga_status s) {
    switch (s) {
        case SVGA_OK: return "ok";
        case SVGA_EINVAL: return "invalid argument";
        case SVGA_EUNSUPPORTED: return "unsupported configuration";
        case SVGA_ECAPACITY: return "buffer too small";
        case SVGA_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* svga_last_error(void) { return g_last_error.c_str(); }

int32_t svga_version(void) { return 104; }

svga_status svga_tilemap_layout(const svga_geom* geom, int32_t bq, int32_t bkv, svga_tilemap_offsets* out) {
    TRY(check_geom(geom));
    TRY(check_tiles(geom, bq, bkv));
    if (!out) return fail(SVGA_EINVAL, "out is NULL");
    MapLayout L = map_layout(geom->F * geom->H * geom->W, bq, bkv);
    out->n_full = L.n_full;
    out->n_bnd = L.n_bnd;
    out->kv = L.kv;
    out->cls = L.cls;
    out->total = L.total;
    out->tq = L.tq;
    out->tk = L.tk;
    return ok();
}

svga_status svga_mask_for_kept_fraction(const svga_geom* geom, int32_t sink_frames, int32_t temporal_layout,
                                        double spatial_target, double temporal_target, svga_mask* out,
                                        int64_t* kept_pairs) {
    TRY(check_geom(geom));
    if (!out) return fail(SVGA_EINVAL, "out is NULL");
    if (!(spatial_target >= 0.0 && spatial_target <= 1.0) || !(temporal_target >= 0.0 && temporal_target <= 1.0))
        return fail(SVGA_EINVAL, "targets must be in [0, 1] (got %g, %g)", spatial_target, temporal_target);
    svga_mask m{sink_frames, 0, 0, temporal_layout};
    TRY(check_mask(&m, geom));
    const int64_t S = (int64_t)geom->H * geom->W;
    m.spatial_band = band_for_kept_fraction(SVGA_KIND_SPATIAL, geom->F, S, sink_frames, spatial_target);
    m.temporal_band = band_for_kept_fraction(SVGA_KIND_TEMPORAL, geom->F, S, sink_frames, temporal_target);
    *out = m;
    if (kept_pairs) {
        kept_pairs[0] = kept_pairs_spatial(geom->F, S, sink_frames, m.spatial_band);
        kept_pairs[1] = kept_pairs_temporal(geom->F, S, sink_frames, m.temporal_band);
    }
    return ok();
}

svga_status svga_build_tilemap_host(const svga_geom* geom, const svga_mask* mask, int32_t bq, int32_t bkv,
                                    int32_t mode, void* h_map, size_t map_bytes) {
    TRY(check_geom(geom));
    TRY(check_mask(mask, geom));
    TRY(check_tiles(geom, bq, bkv));
    TRY(check_mode(mode));
    if (!h_map) return fail(SVGA_EINVAL, "h_map is NULL");
    Geo g = make_geo(*geom, *mask);
    MapLayout L = map_layout(g.N, bq, bkv);
    if (map_bytes < L.total) return fail(SVGA_ECAPACITY, "map_bytes %zu < required %zu", map_bytes, L.total);
    unsigned char* m = static_cast<unsigned char*>(h_map);
    std::memset(m, 0, L.total);
    svga_tilemap_header hdr = map_header(*geom, *mask, bq, bkv, mode, L);
    std::memcpy(m, &hdr, sizeof hdr);
    build_tilemap_host(g, bq, bkv, mode, m, L);
    return ok();
}

svga_status svga_build_tilemap(const svga_geom* geom, const svga_mask* mask, int32_t bq, int32_t bkv, int32_t mode,
                               void* d_map, size_t map_bytes, void* stream) {
    TRY(check_geom(geom));
    TRY(check_mask(mask, geom));
    TRY(check_tiles(geom, bq, bkv));
    TRY(check_mode(mode));
    if (!d_map) return fail(SVGA_EINVAL, "d_map is NULL");
    Geo g = make_geo(*geom, *mask);
    MapLayout L = map_layout(g.N, bq, bkv);
    if (map_bytes < L.total) return fail(SVGA_ECAPACITY, "map_bytes %zu < required %zu", map_bytes, L.total);
    if (L.tk > 8000) return fail(SVGA_EUNSUPPORTED, "device builder needs tk <= 8000 (got %d); use the host builder", L.tk);
    svga_tilemap_header hdr = map_header(*geom, *mask, bq, bkv, mode, L);
    (void)hipGetLastError();
    hipError_t e = launch_build_tilemap(g, bq, bkv, mode, static_cast<unsigned char*>(d_map), L, hdr,
                                        static_cast<hipStream_t>(stream));
    return launched(e, "svga_build_tilemap");
}

static svga_status permute_common(const void* d_in, void* d_out, const uint8_t* d_flags, int32_t B, int32_t n_heads,
                                  const svga_geom* geom, const svga_mask* mask, int32_t head_dim, void* stream,
                                  bool inverse) {
    TRY(check_geom(geom));
    TRY(check_mask(mask, geom));
    TRY(check_heads(B, n_heads));
    if (!d_in || !d_out || !d_flags) return fail(SVGA_EINVAL, "d_in, d_out and d_flags must be non-NULL");
    if (d_in == d_out) return fail(SVGA_EINVAL, "permutation is out of place: d_in == d_out");
    if (head_dim < 8 || head_dim > 512 || head_dim % 8) return fail(SVGA_EINVAL, "head_dim must be a multiple of 8 in [8, 512]");
    const int64_t head_vecs = (int64_t)geom->F * geom->H * geom->W * (head_dim / 8);
    if (head_vecs >= (int64_t(1) << 31))
        return fail(SVGA_EINVAL, "N * head_dim / 8 = %lld must be below 2^31", (long long)head_vecs);
    Geo g = make_geo(*geom, *mask);
    (void)hipGetLastError();
    hipError_t e = launch_permute(d_in, d_out, d_flags, B * n_heads, g, head_dim, inverse, static_cast<hipStream_t>(stream));
    return launched(e, inverse ? "svga_unpermute" : "svga_permute");
}

svga_status svga_permute(const void* d_in, void* d_out, const uint8_t* d_flags, int32_t B, int32_t n_heads,
                         const svga_geom* geom, const svga_mask* mask, int32_t head_dim, void* stream) {
    return permute_common(d_in, d_out, d_flags, B, n_heads, geom, mask, head_dim, stream, false);
}

svga_status svga_unpermute(const void* d_in, void* d_out, const uint8_t* d_flags, int32_t B, int32_t n_heads,
                           const svga_geom* geom, const svga_mask* mask, int32_t head_dim, void* stream) {
    return permute_common(d_in, d_out, d_flags, B, n_heads, geom, mask, head_dim, stream, true);
}

svga_status svga_route_workspace_bytes(int32_t B, int32_t n_heads, const svga_geom* geom, int32_t head_dim,
                                       int32_t n_samples, size_t* bytes) {
    TRY(check_geom(geom));
    TRY(check_heads(B, n_heads));
    if (!bytes) return fail(SVGA_EINVAL, "bytes is NULL");
    if (head_dim != 64 && head_dim != 128) return fail(SVGA_EUNSUPPORTED, "routing supports head_dim 64 or 128");
    if (n_samples < 1 || n_samples > 64) return fail(SVGA_EUNSUPPORTED, "n_samples must be in [1, 64]");
    int32_t chunk, n_chunks;
    route_plan(B * n_heads, geom->F * geom->H * geom->W, head_dim, n_samples, &chunk, &n_chunks, bytes);
    return ok();
}

svga_status svga_route_heads(const void* d_q, const void* d_k, const void* d_v, int32_t B, int32_t n_heads,
                             const svga_geom* geom, const svga_mask* mask, int32_t head_dim,
                             const int32_t* d_sample_idx, int32_t n_samples, float softmax_scale, void* d_workspace,
                             size_t workspace_bytes, uint8_t* d_flags_out, float* d_err_out, void* stream) {
    TRY(check_geom(geom));
    TRY(check_mask(mask, geom));
    TRY(check_heads(B, n_heads));
    if (!d_q || !d_k || !d_v || !d_sample_idx || !d_workspace || !d_flags_out)
        return fail(SVGA_EINVAL, "d_q, d_k, d_v, d_sample_idx, d_workspace and d_flags_out must be non-NULL");
    if (head_dim != 64 && head_dim != 128) return fail(SVGA_EUNSUPPORTED, "routing supports head_dim 64 or 128");
    if (n_samples < 1 || n_samples > 64) return fail(SVGA_EUNSUPPORTED, "n_samples must be in [1, 64]");
    if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return fail(SVGA_EINVAL, "softmax_scale must be finite and > 0");
    RouteLaunch a{};
    size_t need = 0;
    route_plan(B * n_heads, geom->F * geom->H * geom->W, head_dim, n_samples, &a.chunk, &a.n_chunks, &need);
    if (workspace_bytes < need) return fail(SVGA_ECAPACITY, "workspace_bytes %zu < required %zu", workspace_bytes, need);
    a.q = d_q;
    a.k = d_k;
    a.v = d_v;
    a.idx = d_sample_idx;
    a.n_samples = n_samples;
    a.BH = B * n_heads;
    a.head_dim = head_dim;
    a.geo = make_geo(*geom, *mask);
    a.scale = softmax_scale;
    a.ws = d_workspace;
    a.flags = d_flags_out;
    a.err = d_err_out;
    (void)hipGetLastError();
    return launched(launch_route(a, static_cast<hipStream_t>(stream)), "svga_route_heads");
}

static svga_status attn_common(const char* who, const void* d_q, const void* d_k, const void* d_v, void* d_o,
                               float* d_lse, int32_t B, int32_t n_heads, const svga_geom* geom, const svga_mask* mask,
                               int32_t head_dim, float softmax_scale, const uint8_t* d_flags, const void* d_map,
                               size_t map_bytes, int32_t bq, int32_t bkv, int32_t mode, int32_t gather_temporal,
                               int32_t* d_counter, int32_t split, void* stream, bool check_only = false) {
    TRY(check_geom(geom));
    TRY(check_mask(mask, geom));
    TRY(check_heads(B, n_heads));
    TRY(check_tiles(geom, bq, bkv));
    TRY(check_mode(mode));
    if (!d_q || !d_k || !d_v || !d_o || !d_flags || !d_map)
        return fail(SVGA_EINVAL, "d_q, d_k, d_v, d_o, d_flags and d_map must be non-NULL");
    if (d_o == d_q || d_o == d_k || d_o == d_v) return fail(SVGA_EINVAL, "d_o must not alias d_q, d_k or d_v");
    if (gather_temporal != 0 && gather_temporal != 1) return fail(SVGA_EINVAL, "gather_temporal must be 0 or 1");
    if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return fail(SVGA_EINVAL, "softmax_scale must be finite and > 0");
    if (!attn_supported(head_dim, bq, bkv))
        return fail(SVGA_EUNSUPPORTED, "no attention kernel for head_dim=%d bq=%d bkv=%d", head_dim, bq, bkv);
    {
        const int64_t head_bytes = (int64_t)geom->F * geom->H * geom->W * head_dim * 2;
        if (head_bytes >= (int64_t(1) << 31))
            return fail(SVGA_EUNSUPPORTED, "one head of K or V (N * head_dim * 2 = %lld bytes) must be below 2^31 bytes",
                        (long long)head_bytes);
    }
    Geo g = make_geo(*geom, *mask);
    MapLayout L = map_layout(g.N, bq, bkv);
    if (map_bytes < L.total) return fail(SVGA_ECAPACITY, "map_bytes %zu < required %zu", map_bytes, L.total);
    if (check_only) return SVGA_OK;
    AttnLaunch a{};
    a.q = d_q;
    a.k = d_k;
    a.v = d_v;
    a.o = d_o;
    a.lse = d_lse;
    a.flags = d_flags;
    a.map = static_cast<const unsigned char*>(d_map);
    a.L = L;
    a.geo = g;
    a.BH = B * n_heads;
    a.head_dim = head_dim;
    a.bq = bq;
    a.bkv = bkv;
    a.mode = mode;
    a.gather = gather_temporal;
    a.scale = softmax_scale;
    a.counter = d_counter;
    a.split = split;
    bool sup = true;
    (void)hipGetLastError();
    hipError_t e = launch_attn_fwd(a, static_cast<hipStream_t>(stream), &sup);
    if (!sup) return fail(SVGA_EUNSUPPORTED, "no attention kernel for head_dim=%d bq=%d bkv=%d", head_dim, bq, bkv);
    return launched(e, who);
}


svga_status svga_sparse_attn_fwd(const void* d_q, const void* d_k, const void* d_v, void* d_o, float* d_lse,
                                 int32_t B, int32_t n_heads, const svga_geom* geom, const svga_mask* mask,
                                 int32_t head_dim, float softmax_scale, const uint8_t* d_flags, const void* d_map,
                                 size_t map_bytes, int32_t bq, int32_t bkv, int32_t mode, int32_t gather_temporal,
                                 void* stream) {
    return attn_common("svga_sparse_attn_fwd", d_q, d_k, d_v, d_o, d_lse, B, n_heads, geom, mask, head_dim,
                       softmax_scale, d_flags, d_map, map_bytes, bq, bkv, mode, gather_temporal, nullptr, 0, stream);
}

svga_status svga_attn_workspace_bytes(size_t* bytes) {
    if (!bytes) return fail(SVGA_EINVAL, "bytes is NULL");
    *bytes = kAttnWorkspaceBytes;
    return ok();
}

svga_status svga_attn_split_workspace_bytes(int32_t head_dim, int32_t bq, size_t* bytes) {
    if (!bytes) return fail(SVGA_EINVAL, "bytes is NULL");
    if (!attn_supported(head_dim, bq, 128))
        return fail(SVGA_EUNSUPPORTED, "no attention kernel for head_dim=%d bq=%d", head_dim, bq);
    *bytes = attn_split_workspace_bytes(head_dim, bq);
    return ok();
}

svga_status svga_sparse_attn_fwd_ws(const void* d_q, const void* d_k, const void* d_v, void* d_o, float* d_lse,
                                    int32_t B, int32_t n_heads, const svga_geom* geom, const svga_mask* mask,
                                    int32_t head_dim, float softmax_scale, const uint8_t* d_flags, const void* d_map,
                                    size_t map_bytes, int32_t bq, int32_t bkv, int32_t mode, int32_t gather_temporal,
                                    void* d_workspace, size_t workspace_bytes, void* stream) {
    if (!d_workspace) return fail(SVGA_EINVAL, "d_workspace is NULL");
    if (workspace_bytes < kAttnWorkspaceBytes)
        return fail(SVGA_ECAPACITY, "workspace_bytes %zu < required %zu", workspace_bytes, kAttnWorkspaceBytes);
    if (reinterpret_cast<uintptr_t>(d_workspace) % 16 != 0)
        return fail(SVGA_EINVAL, "d_workspace must be 16-byte aligned");
    const int32_t split = attn_supported(head_dim, bq, bkv) && bq >= 32 * kSplitWaves &&
                                  workspace_bytes >= attn_split_workspace_bytes(head_dim, bq)
                              ? 1
                              : 0;
    return attn_common("svga_sparse_attn_fwd_ws", d_q, d_k, d_v, d_o, d_lse, B, n_heads, geom, mask, head_dim,
                       softmax_scale, d_flags, d_map, map_bytes, bq, bkv, mode, gather_temporal,
                       static_cast<int32_t*>(d_workspace), split, stream);
}

svga_status svga_sparse_attn_fwd_noalloc(const void* d_q, const void* d_k, const void* d_v, void* d_o, float* d_lse,
                                         int32_t B, int32_t n_heads, const svga_geom* geom, const svga_mask* mask,
                                         int32_t head_dim, float softmax_scale, const uint8_t* d_flags,
                                         const void* d_map, size_t map_bytes, int32_t bq, int32_t bkv, int32_t mode,
                                         int32_t gather_temporal, void* stream) {
    // the scratch needs of a call depend on head_dim and bq only; every supported pair fits
    if (attn_supported(head_dim, bq, bkv) && attn_split_workspace_bytes(head_dim, bq) > kNoAllocScratchBytes)
        return fail(SVGA_ECAPACITY, "head_dim=%d bq=%d needs %zu scratch bytes, more than the %zu this entry point holds",
                    head_dim, bq, attn_split_workspace_bytes(head_dim, bq), kNoAllocScratchBytes);
    // argument checks first, so that an invalid call touches no device state
    {
        svga_status st = attn_common("svga_sparse_attn_fwd_noalloc", d_q, d_k, d_v, d_o, d_lse, B, n_heads, geom,
                                     mask, head_dim, softmax_scale, d_flags, d_map, map_bytes, bq, bkv, mode,
                                     gather_temporal, nullptr, 0, nullptr, /*check_only=*/true);
        if (st != SVGA_OK) return st;
    }
    void* scratch = nullptr;
    (void)hipGetLastError();
    hipError_t e = noalloc_scratch(&scratch);
    if (e != hipSuccess) return fail(SVGA_EHIP, "svga_sparse_attn_fwd_noalloc: scratch lookup: %s", hipGetErrorString(e));
    const int32_t split = attn_supported(head_dim, bq, bkv) && bq >= 32 * kSplitWaves ? 1 : 0;
    return attn_common("svga_sparse_attn_fwd_noalloc", d_q, d_k, d_v, d_o, d_lse, B, n_heads, geom, mask, head_dim,
                       softmax_scale, d_flags, d_map, map_bytes, bq, bkv, mode, gather_temporal,
                       static_cast<int32_t*>(scratch), split, stream, false);
}

}  // extern "C"

