// Host tile-map builder.
//
// ASTA section "Logical sparsity is not physical sparsity": a tile is full
// (every pair kept), boundary (some kept) or skipped (none kept); section
// "Avoid intra-tile masking when there is nothing to mask": the classes are
// found before attention runs. The count of kept pairs of every tile comes
// from each row's kept key ranges: partial key tiles at a range's two ends get
// the exact overlap, key tiles fully inside a range are counted through a
// difference array over key tiles. All arithmetic is exact integer arithmetic.
#include <algorithm>
#include <cstring>
#include <vector>

#include "svga_internal.h"

namespace svga {

namespace {

struct Counter {
    const Geo& g;
    int32_t bkv;
    bool periodic;
    std::vector<int64_t>& cnt;
    std::vector<int64_t>& diff;

    int64_t psub(int32_t x, int32_t y) const {
        return periodic ? (int64_t)periodic_prefix(g, y) - periodic_prefix(g, x) : 0;
    }

    void add_range(int32_t a, int32_t b) {
        if (a >= b) return;
        int32_t ja = a / bkv, jb = (b - 1) / bkv;
        if (ja == jb) {
            cnt[ja] += (b - a) - psub(a, b);
            return;
        }
        int32_t ea = (ja + 1) * bkv, sb = jb * bkv;
        cnt[ja] += (ea - a) - psub(a, ea);
        cnt[jb] += (b - sb) - psub(sb, b);
        if (jb > ja + 1) {
            diff[ja + 1] += 1;
            diff[jb] -= 1;
        }
    }
};

}  // namespace

void build_tilemap_host(const Geo& g, int32_t bq, int32_t bkv, int32_t mode, unsigned char* h_map,
                        const MapLayout& L) {
    const int32_t N = g.N, tq = L.tq, tk = L.tk;
    std::vector<int64_t> cnt(tk), diff(tk + 1), sp(tk);
    std::vector<int32_t> list_full, list_bnd;
    list_full.reserve(tk);
    list_bnd.reserve(tk);
    for (int kind = 0; kind < 2; ++kind) {
        int32_t* n_full = reinterpret_cast<int32_t*>(h_map + L.n_full) + (size_t)kind * tq;
        int32_t* n_bnd = reinterpret_cast<int32_t*>(h_map + L.n_bnd) + (size_t)kind * tq;
        int32_t* kv = reinterpret_cast<int32_t*>(h_map + L.kv) + (size_t)kind * tq * tk;
        int8_t* cls = reinterpret_cast<int8_t*>(h_map + L.cls) + (size_t)kind * tq * tk;
        const bool periodic = kind == SVGA_KIND_TEMPORAL && g.layout == SVGA_TL_LITERAL && g.k > 0;
        for (int32_t J = 0; J < tk; ++J) {
            int32_t c0 = J * bkv, c1 = std::min(N, (J + 1) * bkv);
            sp[J] = periodic ? (int64_t)periodic_prefix(g, c1) - periodic_prefix(g, c0) : 0;
        }
        Counter ctr{g, bkv, periodic, cnt, diff};
        for (int32_t I = 0; I < tq; ++I) {
            const int32_t r0 = I * bq, r1 = std::min(N, r0 + bq), rows = r1 - r0;
            std::fill(cnt.begin(), cnt.end(), 0);
            std::fill(diff.begin(), diff.end(), 0);
            if (mode != SVGA_MAP_DENSE) {
                for (int32_t i = r0; i < r1; ++i) {
                    RowKeys rk = row_keys(g, kind, i);
                    ctr.add_range(rk.a0, rk.b0);
                    ctr.add_range(rk.a1, rk.b1);
                }
            }
            list_full.clear();
            list_bnd.clear();
            int64_t full_rows = 0;
            for (int32_t J = 0; J < tk; ++J) {
                const int32_t cols = std::min(N, (J + 1) * bkv) - J * bkv;
                full_rows += diff[J];
                const int64_t area = (int64_t)rows * cols;
                int64_t c = area;
                if (mode != SVGA_MAP_DENSE) c = cnt[J] + full_rows * (cols - sp[J]) + (int64_t)rows * sp[J];
                const bool pad_col = (int64_t)(J + 1) * bkv > N;
                const int8_t k = classify_tile(mode, c, area, pad_col);
                cls[(size_t)I * tk + J] = k;
                if (k == SVGA_TILE_FULL) list_full.push_back(J);
                if (k == SVGA_TILE_BOUNDARY) list_bnd.push_back(J);
            }
            int32_t* row = kv + (size_t)I * tk;
            std::copy(list_full.begin(), list_full.end(), row);
            std::copy(list_bnd.begin(), list_bnd.end(), row + list_full.size());
            std::fill(row + list_full.size() + list_bnd.size(), row + tk, -1);
            n_full[I] = (int32_t)list_full.size();
            n_bnd[I] = (int32_t)list_bnd.size();
        }
    }
}

}  // namespace svga
