// Sampled-query head routing for gfx950.
//
// ASTA section "Speeding up attention": Sparse VideoGen samples a few
// queries per head, computes their outputs under dense, spatial and temporal
// attention, and routes the head to the sparse mask whose output deviates
// least from the dense one; section "Support dynamic routing with fixed
// tensor shapes": the result is a Boolean flag per head that stays on the
// device.
//
// Pass 1 (route_partial_kernel): one workgroup per (batch*head, key chunk).
// Each wave holds 32 sampled queries as MFMA B operands and runs one of the
// three softmaxes (dense, spatial mask, temporal mask) with its own running
// max, sum and output; every K/V sub-tile of the chunk is staged through LDS
// once and serves all waves. The softmax kind is wave-uniform, so each wave
// runs a loop specialised to it; its mask is a 64-bit keep mask over the
// step's keys (built from at most two key ranges, or from the frames the step
// touches) and costs a bit test per score. P is split into a bf16 high part
// and a bf16 remainder, both fed to the MFMA, so the weighted sums keep about
// 16 mantissa bits. The partial (max, sum, output) of every softmax is
// written to the workspace.
// Pass 2 (route_merge_kernel): one workgroup per (sample, batch*head) merges
// the chunk partials and forms that sample's ||o_x - o_dense||^2.
// Pass 3 (route_flag_kernel): err_x = sum over samples, in sample order; the
// flag is 1 (temporal) iff err_temporal < err_spatial.
// Memory traffic: K and V read once; roofline is HBM bandwidth.
#include <type_traits>

#include "tile_stage.h"

namespace svga {

namespace {

constexpr int kMaxSamples = 64;

struct RArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* idx;
    int32_t ns, chunk, n_chunks;
    Geo g;
    float c2;
    float* ws;       // [BH][n_chunks][3][kMaxSamples][D + 2]: max (log2 domain), sum, output
    float* ws_err;   // [BH][kMaxSamples][2]: per-sample squared deviations (spatial, temporal)
    uint8_t* flags;
    float* err;
};

template <int D>
__device__ __forceinline__ size_t ws_index(int bh, int chunk, int n_chunks, int x, int n) {
    return ((((size_t)bh * n_chunks + chunk) * 3 + x) * kMaxSamples + n) * (D + 2);
}

// QBLK blocks of 32 samples; wave w serves sample block w / 3 under softmax
// kind w % 3 (0 dense, 1 spatial mask, 2 temporal mask).
template <int D, int QBLK, int KSUB>
__global__ __launch_bounds__(QBLK * 3 * 64) void route_partial_kernel(RArgs a) {
    constexpr int NT = QBLK * 3 * 64;
    constexpr int KBLK = KSUB / 32;
    constexpr int DB = D / 32;
    constexpr int DC = D / 16;
    using St = Stager<D, KSUB, NT>;
    __shared__ __attribute__((aligned(16))) char smem[2 * St::STAGE];

    const int chunk = blockIdx.x, bh = blockIdx.y;
    const Geo& g = a.g;
    const int N = g.N;
    const int c0 = chunk * a.chunk;
    const int c1 = imin(N, c0 + a.chunk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int x = __builtin_amdgcn_readfirstlane(wave % 3);   // softmax kind of this wave (wave-uniform)
    const size_t head_off = (size_t)bh * N * D;
    const uint16_t* kh = a.k + head_off;
    const uint16_t* vh = a.v + head_off;

    const int n = (wave / 3) * 32 + l32;              // sample slot of this lane
    int qtok = a.idx[imin(n, a.ns - 1)];
    qtok = imin(imax(qtok, 0), N - 1);
    bf16x8 qreg[DC];
    {
        const bf16x8* p = reinterpret_cast<const bf16x8*>(a.q + head_off + (size_t)qtok * D + 8 * h);
#pragma unroll
        for (int c = 0; c < DC; ++c) qreg[c] = p[2 * c];
    }
    const RowKeys rks = row_keys(g, SVGA_KIND_SPATIAL, qtok);   // frame-major = spatial order
    uint32_t fq, sq;
    g.divS.divmod((uint32_t)qtok, fq, sq);

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float mrow = -INFINITY, lrow = 0.f;

    const int steps = (c1 - c0 + KSUB - 1) / KSUB;
    St st;
    auto ident = [](int j) { return j; };
    if (steps > 0) {
        st.load(kh, vh, c0, N, ident, tid);
        st.store(smem, tid);
        if (steps > 1) st.load(kh, vh, c0 + KSUB, N, ident, tid);
    }
    __syncthreads();

    // 64-bit keep mask over keys kb0 .. kb0+63 for this lane's sample under softmax kind X
    // (frame-major coordinates), keys at or past the chunk end excluded
    auto keep_bits = [&](auto X, int kb0) __attribute__((always_inline)) {
        uint64_t m = window_bits(kb0, c1, kb0);
        if constexpr (decltype(X)::value == 1) {
            m &= window_bits(rks.a0, rks.b0, kb0) | window_bits(rks.a1, rks.b1, kb0);
        } else if constexpr (decltype(X)::value == 2) {
            // sink frames whole; in every other frame the positions within bt of the sample's
            uint64_t t = 0;
            const int f0 = kb0 / g.S, f1 = imin((kb0 + KSUB - 1) / g.S, g.F - 1);
            for (int f = f0; f <= f1; ++f) {
                const int fs = f * g.S;
                t |= f < g.k ? window_bits(fs, fs + g.S, kb0)
                             : window_bits(fs + imax((int)sq - g.bt, 0), fs + imin((int)sq + g.bt + 1, g.S), kb0);
            }
            m &= t;
        }
        return m;
    };
    auto run = [&](auto X) __attribute__((always_inline)) {
        for (int s = 0; s < steps; ++s) {
            const char* stg = smem + (s & 1) * St::STAGE;
            const int kb0 = c0 + s * KSUB;
            f32x16 sacc[KBLK];
#pragma unroll
            for (int b = 0; b < KBLK; ++b) sacc[b] = f32x16{};
#pragma unroll
            for (int c = 0; c < DC; ++c)
#pragma unroll
                for (int b = 0; b < KBLK; ++b)
                    sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(St::a_k(stg, b, c, l32, h), qreg[c], sacc[b], 0, 0, 0);

            // mask by a bit test per score: bit acc_key(b, i, 0) - 32 b of word b, after a shift
            // that puts this half-wave's keys at acc_key(b, i, 0)
            const uint64_t m = keep_bits(X, kb0) >> acc_key(0, 0, h);
            const uint32_t mw[2] = {(uint32_t)m, (uint32_t)(m >> 32)};
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < KBLK; ++b) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int pos = acc_key(b, i, 0) - 32 * b;
                    if (!((mw[b] >> pos) & 1u)) sacc[b][i] = -INFINITY;
                    mx = fmaxf(mx, sacc[b][i]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(mrow, mx);
            const float base = mnew == -INFINITY ? 0.f : mnew * a.c2;
            const float alpha = __builtin_amdgcn_exp2f(mrow * a.c2 - base);
            mrow = mnew;
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            const int vlo = St::v_lane_off(lane);
#pragma unroll
            for (int m16 = 0; m16 < KSUB / 16; ++m16) {
                // registers 8*(m16%2) .. +7 of key block m16/2 hold keys 16*m16 + 8h .. +7
                bf16x8 hi8, lo8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[m16 >> 1][8 * (m16 & 1) + e], a.c2, -base));
                    lrow += p;
                    const __bf16 ph = (__bf16)p;
                    hi8[e] = ph;
                    lo8[e] = (__bf16)(p - (float)ph);
                }
                bf16x8 av[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) av[db] = St::a_v(stg, db, m16, vlo);
                // the high parts of all dimension blocks, then the low parts: no product
                // waits on the one just before it
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[db], hi8, oacc[db], 0, 0, 0);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[db], lo8, oacc[db], 0, 0, 0);
            }

            if (s + 1 < steps) {
                st.store(smem + ((s + 1) & 1) * St::STAGE, tid);
                if (s + 2 < steps) st.load(kh, vh, kb0 + 2 * KSUB, N, ident, tid);
            }
            __syncthreads();
        }
    };
    // the kind is uniform per wave, so each wave runs one specialised loop (all pass the same barriers)
    if (x == 0) run(std::integral_constant<int, 0>{});
    else if (x == 1) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 2>{});

    // ---- partial of this (sample, kind): max in the log2 domain, sum, unnormalised output
    const float lt = lrow + __shfl_xor(lrow, 32);
    float* w = a.ws + ws_index<D>(bh, chunk, a.n_chunks, x, n);
    if (h == 0) {
        w[0] = mrow == -INFINITY ? -INFINITY : mrow * a.c2;
        w[1] = lt;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) w[2 + db * 32 + 8 * (i >> 2) + 4 * h + (i & 3)] = oacc[db][i];
}

// One workgroup (D threads) per (sample, batch*head): merge the chunk partials
// of the three softmaxes, then this sample's two squared deviations.
template <int D>
__global__ __launch_bounds__(D) void route_merge_kernel(RArgs a) {
    const int n = blockIdx.x, bh = blockIdx.y;
    const int t = threadIdx.x;
    __shared__ float red[3][D];
    __shared__ float Mx[3], Lx[3];
    // running maxima of the three softmaxes over chunks
    float m3[3] = {-INFINITY, -INFINITY, -INFINITY};
    for (int c = t; c < a.n_chunks; c += D)
#pragma unroll
        for (int x = 0; x < 3; ++x) m3[x] = fmaxf(m3[x], a.ws[ws_index<D>(bh, c, a.n_chunks, x, n)]);
#pragma unroll
    for (int x = 0; x < 3; ++x) red[x][t] = m3[x];
    __syncthreads();
    for (int w = D / 2; w > 0; w >>= 1) {
        if (t < w)
#pragma unroll
            for (int x = 0; x < 3; ++x) red[x][t] = fmaxf(red[x][t], red[x][t + w]);
        __syncthreads();
    }
    if (t < 3) Mx[t] = red[t][0];
    __syncthreads();
    float l3[3] = {0.f, 0.f, 0.f};
    for (int c = t; c < a.n_chunks; c += D)
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const float* w = a.ws + ws_index<D>(bh, c, a.n_chunks, x, n);
            if (Mx[x] != -INFINITY) l3[x] += w[1] * __builtin_amdgcn_exp2f(w[0] - Mx[x]);
        }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 3; ++x) red[x][t] = l3[x];
    __syncthreads();
    for (int w = D / 2; w > 0; w >>= 1) {
        if (t < w)
#pragma unroll
            for (int x = 0; x < 3; ++x) red[x][t] += red[x][t + w];
        __syncthreads();
    }
    if (t < 3) Lx[t] = red[t][0];
    __syncthreads();
    // the three softmaxes' chunk loops fused, loads issued unconditionally and
    // eight chunks ahead so that they overlap (each sum still runs in chunk
    // order; a softmax whose max is -inf has no kept key and contributes 0)
    float acc[3] = {0.f, 0.f, 0.f};
    float mb[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) mb[x] = Mx[x] == -INFINITY ? 0.f : Mx[x];
    constexpr size_t XS = (size_t)kMaxSamples * (D + 2);   // stride between the three softmaxes' partials
    const float* w0 = a.ws + ws_index<D>(bh, 0, a.n_chunks, 0, n);
    constexpr size_t CS = 3 * XS;                           // stride between chunks
#pragma unroll 8
    for (int c = 0; c < a.n_chunks; ++c) {
        const float* w = w0 + (size_t)c * CS;
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const float e = w[x * XS + 2 + t] * __builtin_amdgcn_exp2f(w[x * XS] - mb[x]);
            acc[x] += Mx[x] != -INFINITY ? e : 0.f;
        }
    }
    float o[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) o[x] = Lx[x] > 0.f ? acc[x] / Lx[x] : 0.f;
    __syncthreads();
    red[0][t] = (o[1] - o[0]) * (o[1] - o[0]);
    red[1][t] = (o[2] - o[0]) * (o[2] - o[0]);
    __syncthreads();
    for (int w = D / 2; w > 0; w >>= 1) {
        if (t < w) {
            red[0][t] += red[0][t + w];
            red[1][t] += red[1][t + w];
        }
        __syncthreads();
    }
    if (t == 0) {
        float* e = a.ws_err + ((size_t)bh * kMaxSamples + n) * 2;
        e[0] = red[0][0];
        e[1] = red[1][0];
    }
}

// One thread per batch*head: sum the per-sample deviations in sample order, set the flag.
__global__ void route_flag_kernel(RArgs a, int BH) {
    const int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    float es = 0.f, et = 0.f;
    for (int n = 0; n < a.ns; ++n) {
        es += a.ws_err[((size_t)bh * kMaxSamples + n) * 2];
        et += a.ws_err[((size_t)bh * kMaxSamples + n) * 2 + 1];
    }
    a.flags[bh] = et < es ? 1 : 0;
    if (a.err) {
        a.err[2 * bh] = es;
        a.err[2 * bh + 1] = et;
    }
}

template <int D, int QBLK, int KSUB>
hipError_t launch_pair(const RArgs& r, int BH, hipStream_t stream) {
    hipLaunchKernelGGL((route_partial_kernel<D, QBLK, KSUB>), dim3(r.n_chunks, BH), dim3(QBLK * 3 * 64), 0, stream, r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_merge_kernel<D>), dim3(r.ns, BH), dim3(D), 0, stream, r);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_flag_kernel, dim3((BH + 63) / 64), dim3(64), 0, stream, r, BH);
    return hipGetLastError();
}

}  // namespace

void route_plan(int32_t BH, int32_t N, int32_t head_dim, int32_t n_samples, int32_t* chunk, int32_t* n_chunks,
                size_t* ws_bytes) {
    (void)n_samples;
    // About 512 workgroups in all, chunks a multiple of 64 keys. Fewer, longer
    // chunks keep the partials small (each chunk writes 3 x 64 rows of D + 2
    // floats per head, which the merge reads back), more chunks spread the
    // pass better: measured fastest among 256 .. 2048 workgroups at 75,600
    // and 302,400 tokens (at 75,600: 256 -> 0.29 ms, 384 -> 0.22, 512 -> 0.19,
    // 768 -> 0.20 for the partial pass).
    int64_t target = ((int64_t)N * BH + 511) / 512;
    int64_t c = (target + 63) / 64 * 64;
    if (c < 256) c = 256;
    *chunk = (int32_t)c;
    *n_chunks = (int32_t)((N + c - 1) / c);
    *ws_bytes = ((size_t)BH * (size_t)*n_chunks * 3 * kMaxSamples * (size_t)(head_dim + 2) +
                 (size_t)BH * kMaxSamples * 2) * sizeof(float);
}

hipError_t launch_route(const RouteLaunch& a, hipStream_t stream) {
    RArgs r;
    r.q = static_cast<const uint16_t*>(a.q);
    r.k = static_cast<const uint16_t*>(a.k);
    r.v = static_cast<const uint16_t*>(a.v);
    r.idx = a.idx;
    r.ns = a.n_samples;
    r.chunk = a.chunk;
    r.n_chunks = a.n_chunks;
    r.g = a.geo;
    r.c2 = a.scale * 1.4426950408889634f;
    r.ws = static_cast<float*>(a.ws);
    r.ws_err = r.ws + (size_t)a.BH * a.n_chunks * 3 * kMaxSamples * (a.head_dim + 2);
    r.flags = a.flags;
    r.err = a.err;
    const bool two = a.n_samples > 32;
    if (a.head_dim == 64) return two ? launch_pair<64, 2, 64>(r, a.BH, stream) : launch_pair<64, 1, 64>(r, a.BH, stream);
    return two ? launch_pair<128, 2, 64>(r, a.BH, stream) : launch_pair<128, 1, 64>(r, a.BH, stream);
}

}  // namespace svga
