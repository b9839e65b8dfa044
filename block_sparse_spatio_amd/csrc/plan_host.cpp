// Host-side planning of libsvga: which attention tile shapes have kernels,
// how routing splits the keys, and the kept-pair counts of the masks with the
// band that meets a target kept fraction. No HIP calls.
#include <cmath>

#include "svga_internal.h"

namespace svga {

bool attn_supported(int32_t head_dim, int32_t bq, int32_t bkv) {
    if (head_dim != 64 && head_dim != 128) return false;
    if (!(bq == 32 || bq == 64 || bq == 128 || bq == 256 || bq == 512)) return false;
    return bkv >= 32 && bkv <= 512 && bkv % 32 == 0;
}

void route_plan(int32_t BH, int32_t N, int32_t head_dim, int32_t n_samples, int32_t* chunk, int32_t* n_chunks,
                size_t* ws_bytes) {
    (void)n_samples;
    // About one workgroup per CU of MI355X (256 in all, whole chunks per
    // head), each chunk a multiple of two 64-key halves: every CU then reads
    // its share of K and V once, and the partials (3 x 64 rows of D + 2
    // floats per chunk) stay about 0.1 MB per workgroup.
    const int64_t per_head = BH >= 256 ? 1 : 256 / BH;
    int64_t c = ((int64_t)N + per_head - 1) / per_head;
    c = (c + 127) / 128 * 128;
    *chunk = (int32_t)c;
    *n_chunks = (int32_t)((N + c - 1) / c);
    *ws_bytes = ((size_t)BH * (size_t)*n_chunks * 3 * kRouteMaxSamples * (size_t)(head_dim + 2) +
                 (size_t)BH * kRouteMaxSamples * 2) * sizeof(float);
}

// Kept (query, key) pairs of a whole head, from the mask definitions of ASTA
// section "Speeding up attention" (Figure 3), counted per query frame or per
// spatial position; the token order does not change them.
int64_t kept_pairs_spatial(int32_t F, int64_t S, int32_t sink, int32_t band) {
    // query frame f keeps the frames of [f - band, f + band] within [0, F),
    // plus the sink frames outside that range: S * S pairs per kept frame
    int64_t frames = 0;
    for (int32_t f = 0; f < F; ++f) {
        const int32_t lo = f - band < 0 ? 0 : f - band;
        const int32_t hi = (int64_t)f + band > F - 1 ? F - 1 : f + band;
        frames += (hi - lo + 1) + (sink < lo ? sink : lo) + (sink - 1 - hi > 0 ? sink - 1 - hi : 0);
    }
    return frames * S * S;
}

int64_t kept_pairs_temporal(int32_t F, int64_t S, int32_t sink, int32_t band) {
    // per frame, sum over query positions s of |{s' in [0, S) : |s' - s| <= band}|:
    // S (2 band + 1) less the band (band + 1) / 2 positions cut at each end
    const int64_t w = band < S - 1 ? band : S - 1;
    const int64_t window_sum = S * (2 * w + 1) - w * (w + 1);
    // every query keeps the sink frames whole and its window in each other frame
    return (int64_t)F * ((int64_t)sink * S * S + (int64_t)(F - sink) * window_sum);
}

// Smallest band whose kept pairs reach target * N^2, the comparison exact:
// target = m 2^-sh with m a 53-bit integer, so the least integer count
// meeting it is ceil(m N^2 / 2^sh), formed in 128-bit arithmetic. Bands run
// up to the first that keeps every pair (F - 1 frames, S - 1 positions).
int32_t band_for_kept_fraction(int32_t kind, int32_t F, int64_t S, int32_t sink, double target) {
    const unsigned __int128 n2 = (unsigned __int128)((int64_t)F * S) * (unsigned __int128)((int64_t)F * S);
    int e = 0;
    const double frac = std::frexp(target, &e);              // target = frac 2^e, frac in [0.5, 1)
    const uint64_t m = (uint64_t)std::ldexp(frac, 53);       // exact
    const int sh = 53 - e;                                   // >= 52 for target <= 1
    const unsigned __int128 prod = (unsigned __int128)m * n2;
    unsigned __int128 need;
    if (target <= 0.0) need = 0;
    else if (sh >= 120) need = prod > 0 ? 1 : 0;
    else need = (prod + (((unsigned __int128)1 << sh) - 1)) >> sh;
    const int32_t last = kind == SVGA_KIND_SPATIAL ? F - 1 : (int32_t)(S - 1);
    // kept pairs grow with the band: bisect for the first band that reaches need
    int32_t lo = 0, hi = last;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        const int64_t kept = kind == SVGA_KIND_SPATIAL ? kept_pairs_spatial(F, S, sink, mid)
                                                       : kept_pairs_temporal(F, S, sink, mid);
        if ((unsigned __int128)kept >= need) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

}  // namespace svga
