// Sampled-query head routing for gfx950.
//
// ASTA section "Speeding up attention": Sparse VideoGen samples a few
// queries per head, computes their outputs under dense, spatial and temporal
// attention, and routes the head to the sparse mask whose output deviates
// least from the dense one; section "Support dynamic routing with fixed
// tensor shapes": the result is a Boolean flag per head that stays on the
// device.
//
// Pass 1 (route_partial_kernel): one workgroup per (batch*head, key chunk),
// about one per CU in all. The chunk is split in two halves, each walked by
// its own waves over its own double-buffered LDS stage; each wave holds 32
// sampled queries as MFMA B operands. Per step of KSUB keys a wave computes
// the scores S^T = K Q^T once and feeds all three softmaxes (dense, spatial
// mask, temporal mask) from them: the three share one running exponent base
// (the dense running maximum, rescaled lazily), so each score costs one
// exponential, and the masked probabilities are the dense ones with excluded
// keys set to zero. P is split into a bf16 high part and a bf16 remainder,
// both fed to the MFMA, so the weighted sums keep about 16 mantissa bits.
// The spatial mask keeps or drops a sample's keys a whole frame at a time:
// when a key half is no longer than a frame (so it touches at most two
// frames), the dense sums are kept per frame and the spatial ones formed
// from them at the end, which leaves 5 products of 2*d FLOP per (sample,
// key): one for the scores, two (high and low part) for the dense output,
// two for the temporal one. Otherwise each softmax has its own sums (7
// products). Masks are keep masks over the step's keys (from at most two
// key ranges, or from the frames the step touches), a bit test per score.
// At the end the two halves merge in LDS and the workgroup writes one
// partial (exponent base, three sums, three unnormalised outputs) per
// sample.
// Pass 2 (route_merge_kernel): one workgroup per (sample, batch*head) merges
// the chunk partials and forms that sample's ||o_x - o_dense||^2.
// Pass 3 (route_flag_kernel): err_x = sum over samples, in sample order; the
// flag is 1 (temporal) iff err_temporal < err_spatial.
// Memory traffic: K and V read once; roofline is HBM bandwidth.
//
// The shared base is the dense maximum, which is at least each masked
// maximum, so masked probabilities are exact fractions of it; a sample whose
// kept scores all lie more than 126 (in log2 units of the scaled scores)
// below its dense maximum would underflow to an empty masked softmax.
#include <type_traits>

#include "tile_stage.h"

namespace svga {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kMaxSamples = kRouteMaxSamples;
constexpr int kRouteParts = 2;   // key halves per workgroup
constexpr int kRouteBlocks = 4;  // blocks of 16 sampled queries (kMaxSamples = 64)

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

// Bits [a - base, b - base) of a 32-bit mask over keys base .. base+31 (clamped).
__device__ __forceinline__ uint32_t window_bits32(int a, int b, int base) {
    const int lo = imin(imax(a - base, 0), 32), hi = imin(imax(b - base, 0), 32);
    const uint32_t below_hi = hi >= 32 ? ~0u : (1u << hi) - 1u;
    const uint32_t below_lo = lo >= 32 ? ~0u : (1u << lo) - 1u;
    return below_hi & ~below_lo;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reductions over the four lanes l % 16 + 16 j. v_permlane16_swap of x with
// itself leaves, in every lane, the values of rows 2i and 2i+1 (16-lane rows)
// of its pair of rows in its two results; v_permlane32_swap the same for the
// two 32-lane halves. Combining the two results of each swap reduces a level.
__device__ __forceinline__ float group_max(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])));
    const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)t[0]), __builtin_bit_cast(float, (uint32_t)t[1]));
}
__device__ __forceinline__ float group_sum(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
    const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)t[0]) + __builtin_bit_cast(float, (uint32_t)t[1]);
}

// Two bf16 (round to nearest even) packed in one word, x in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    const bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
}

// 0xffff in each half of pair j whose bit (2j, 2j+1) of bits is set: each bit
// sign-extended to a full word, the two words merged by a bitfield insert.
__device__ __forceinline__ uint32_t pair_mask(uint32_t bits, int j) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 2 * j, 1);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 2 * j + 1, 1);
    return (lo & 0x0000ffffu) | (hi & 0xffff0000u);
}

// Sum of the two bf16 halves of each word, accumulated in fp32 (v_dot2 with ones).
__device__ __forceinline__ float pair_sum(const uint32_t (&w)[4], float acc) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w[j]), one, acc, false);
    return acc;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    return __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
}

// New base when the running max grows by more than 2^16. A rescale costs a
// wave 3 x D / 16 x 4 multiplies and any of its 16 samples triggers it, so a
// wide margin pays (4.5% at 75,600 tokens against 2^8): weights stay at or
// below 2^16, so even a chunk of 2^20 keys sums below 2^36, far inside the
// fp32 and bf16 range.
constexpr float kRouteRescaleLog2 = 16.0f;

// Waves: kRouteBlocks blocks of 16 samples x kRouteParts key halves; wave
// w serves sample block w % kRouteBlocks over key half w / kRouteBlocks.
// Products are v_mfma_f32_16x16x32_bf16 (lane l holds row / column l % 16
// and the 8 consecutive reduction elements 8 (l / 16) .. +7 of its A / B
// operand, and rows 4 (l / 16) .. +3 of column l % 16 of the result):
// * S^T = K Q^T in two chains of 16 keys (keys 16 j .. 16 j + 15), so lane
//   group g = l / 16 ends up with the scores of keys 4 g .. 4 g + 3 and
//   16 + 4 g .. + 3 of its sample: the B operand of
// * O^T = V^T P^T per block of 16 dimensions, whose reduction runs over the
//   step's keys in that same order: V^T comes from two transposing LDS reads
//   (keys 4 g .. 4 g + 3 and 16 + 4 g .. + 3).
// Each lane then owns 8 (sample, key) scores per 32-key step and 3 * D / 16
// accumulator registers, so two waves share each SIMD.
template <int D, bool TWO>
__global__ __launch_bounds__(kRouteBlocks * kRouteParts * 64) __attribute__((amdgpu_waves_per_eu(2)))
void route_partial_kernel(RArgs a) {
    constexpr int KSUB = 32;
    constexpr int PT = kRouteBlocks * 64;         // threads of one key half
    constexpr int DB = D / 16;                    // 16-dimension blocks of the output
    constexpr int DC = D / 32;                    // 32-dimension chunks of the scores
    // K rows padded as in the attention kernel; V rows 32 bytes past a
    // multiple of 256, so that the 8 rows of keys 0..7 (one half-wave's
    // transposing read below) start 8 banks apart and never share a bank
    using St = Stager<D, KSUB, PT, 32>;
    constexpr int MERGE_BYTES = kRouteBlocks * 3 * 16 * (D + 2) * 4;
    constexpr int SMEM = kRouteParts * 2 * St::STAGE > MERGE_BYTES ? kRouteParts * 2 * St::STAGE : MERGE_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    const int chunk = blockIdx.x, bh = blockIdx.y;
    const Geo& g = a.g;
    const int N = g.N;
    // the wave index through readfirstlane, so that everything derived from it
    // (key half, step keys, frame ranges) is known wave-uniform and kept in SGPRs
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int part = wave / kRouteBlocks, sb = wave - part * kRouteBlocks;
    const int ptid = tid - part * PT;
    const int l16 = lane & 15, grp = lane >> 4;
    const int sub = a.chunk / kRouteParts;             // a multiple of KSUB
    const int c0 = chunk * a.chunk + part * sub;
    const int c1 = imin(N, c0 + sub);                  // keys of this half: [c0, c1), possibly empty
    const int steps = sub / KSUB;                      // the same for every wave: equal barrier counts
    // TWO (a half no longer than a frame): the half's keys lie in frame fa and
    // possibly fa + 1, from key kbnd on. Sum set 0 then takes the dense terms
    // of the current frame, and when frame fa + 1 begins, frame fa's sums
    // move to set 1; the spatial output is formed at the end from the frames
    // the sample's mask keeps.
    const int fa = (int)g.divS.div((uint32_t)imin(c0, N - 1));
    const int kbnd = (fa + 1) * g.S;
    char* sm = smem + part * 2 * St::STAGE;
    const size_t head_off = (size_t)bh * N * D;
    const uint16_t* kh = a.k + head_off;
    const uint16_t* vh = a.v + head_off;

    const int n = sb * 16 + l16;                       // sample slot of this lane
    int qtok = a.idx[imin(n, a.ns - 1)];
    qtok = imin(imax(qtok, 0), N - 1);
    bf16x8 qreg[DC];   // B operand: dims 32 c + 8 grp .. +7 of the sample
    {
        const uint16_t* p = a.q + head_off + (size_t)qtok * D + 8 * grp;
#pragma unroll
        for (int c = 0; c < DC; ++c) qreg[c] = *reinterpret_cast<const bf16x8*>(p + 32 * c);
    }
    const RowKeys rks = row_keys(g, SVGA_KIND_SPATIAL, qtok);   // frame-major = spatial order
    uint32_t fq, sq;
    g.divS.divmod((uint32_t)qtok, fq, sq);

    // unnormalised outputs and sums: dense, spatial, temporal (TWO: the
    // current frame's dense terms, frame fa's once fa + 1 has begun, temporal)
    f32x4 oacc[3][DB];
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[x][db] = f32x4{};
    float base = -INFINITY;
    float lsum[3] = {0.f, 0.f, 0.f};

    // K / V copy. With few chunks per thread, two register sets, so that the
    // loads of step t are issued two steps before step t - 1 stores them to
    // LDS (set t % 2 holds step t); otherwise one set, loaded one step ahead.
    constexpr bool DEEP = St::CU <= 2;
    constexpr int AHEAD = DEEP ? 3 : 2;
    St st0, st1;
    auto ident = [](int j) { return j; };
    // A chunk is a multiple of 128 keys, so every half has at least 2 steps.
    // No branch around these first copies: the wait for their loads then also
    // covers the Q loads on every path into the loop, so the loop's products
    // on Q carry no wait for the loads in flight.
    st0.load(kh, vh, c0, N, ident, ptid);
    st0.store(sm, ptid);
    (DEEP ? st1 : st0).load(kh, vh, c0 + KSUB, N, ident, ptid);
    if (DEEP && steps > 2) st0.load(kh, vh, c0 + 2 * KSUB, N, ident, ptid);
    __syncthreads();

    // temporal keep mask over the 32 keys base .. base+31: sink frames whole,
    // in every other frame the positions within bt of the sample's
    const int tlo = imax((int)sq - g.bt, 0), thi = imin((int)sq + g.bt + 1, g.S);
    auto temporal_bits = [&](int base_key) __attribute__((always_inline)) {
        uint32_t t = 0;
        const int f0 = (int)g.divS.div((uint32_t)base_key);
        const int f1 = imin((int)g.divS.div((uint32_t)(base_key + 31)), g.F - 1);
        for (int f = f0; f <= f1; ++f) {
            const int fs = f * g.S;
            t |= f < g.k ? window_bits32(fs, fs + g.S, base_key) : window_bits32(fs + tlo, fs + thi, base_key);
        }
        return t;
    };
    // per-lane LDS offsets: K row l16 of the two score chains (16 consecutive
    // rows per read, conflict-free with the padded rows); V^T operand (dims
    // 16 db + 4 (l16 % 4) .. +3 of key 4 grp + l16 / 4, and 16 keys on)
    const int koff0 = l16 * St::KROW + grp * 16, koff1 = koff0 + 16 * St::KROW;
    const int voff = St::KBYTES + (4 * grp + (l16 >> 2)) * St::VROW + (l16 & 3) * 8;
    auto step = [&](const int s, St& nxt) __attribute__((always_inline)) {
        const char* stg = sm + (s & 1) * St::STAGE;
        const int kb0 = c0 + s * KSUB;
        f32x4 sc0 = f32x4{}, sc1 = f32x4{};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(stg + koff0 + c * 64);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(stg + koff1 + c * 64);
            sc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[c], sc0, 0, 0, 0);
            sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[c], sc1, 0, 0, 0);
        }
        // the V^T operands of this step, read now so that the softmax below hides their latency
        bf16x8 av[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const char* vp = stg + voff + db * 32;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 16 * St::VROW));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            av[db] = __builtin_bit_cast(bf16x8, both);
        }
        const bool whole = kb0 + KSUB <= c1;   // wave-uniform: every key of the step is in the half
        // bits of this lane's 8 keys, in element order, of a mask over keys kb0 .. kb0+31
        auto mine = [&](uint32_t m) __attribute__((always_inline)) {
            return __builtin_amdgcn_ubfe(m, 4 * grp, 4) | (__builtin_amdgcn_ubfe(m, 16 + 4 * grp, 4) << 4);
        };
        // Keep bits of the lane's keys. Usually the step lies in one frame f0
        // (wave-uniform): the spatial mask keeps the whole frame or none of it,
        // and the temporal one the sample's window within it, or all of a sink
        // frame. A step across frames takes the general ranges.
        const int f0 = (int)g.divS.div((uint32_t)kb0);
        const bool one_frame = f0 == (int)g.divS.div((uint32_t)(kb0 + KSUB - 1));
        uint32_t bs, bt;
        // TWO: frame fa + 1 begins in this step (wave-uniform); bs marks its keys of frame fa
        const bool cross = TWO && kb0 <= kbnd && kbnd < kb0 + KSUB;
        if constexpr (TWO) {
            bs = cross ? mine(window_bits32(kb0, kbnd, kb0)) : 0xffu;
            bt = one_frame ? (f0 < g.k ? 0xffu : mine(window_bits32(f0 * g.S + tlo, f0 * g.S + thi, kb0)))
                           : mine(temporal_bits(kb0));
        } else if (one_frame) {
            bs = f0 < g.k || abs(f0 - (int)fq) <= g.bs ? 0xffu : 0u;
            bt = f0 < g.k ? 0xffu : mine(window_bits32(f0 * g.S + tlo, f0 * g.S + thi, kb0));
        } else {
            bs = mine(window_bits32(rks.a0, rks.b0, kb0) | window_bits32(rks.a1, rks.b1, kb0));
            bt = mine(temporal_bits(kb0));
        }
        if (!whole) {
            // the step runs over the end of the half (rare): its keys past the end
            // get a score of -inf, so that no softmax keeps them
            const uint32_t bd = mine(window_bits32(kb0, c1, kb0));
            bs &= bd;
            bt &= bd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc0[e] = (bd >> e) & 1u ? sc0[e] : -INFINITY;
                sc1[e] = (bd >> (4 + e)) & 1u ? sc1[e] : -INFINITY;
            }
        }
        // this lane's scores: element e < 4 is key kb0 + 4 grp + e, e >= 4 key kb0 + 12 + 4 grp + e
        const float sc[8] = {sc0[0], sc0[1], sc0[2], sc0[3], sc1[0], sc1[1], sc1[2], sc1[3]};
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc[e]);
        mx = group_max(mx);
        // a new base when this step's max exceeds the current one by more than 2^16
        const float cand = mx * a.c2;
        const bool grow = cand > base + kRouteRescaleLog2;
        if (__any(grow)) {
            // rare after a sample's first steps: kept as a branch (the empty asm
            // stops the compiler from turning it into unconditional multiplies)
            asm volatile("" ::: "memory");
            const float nb = grow ? cand : base;
            const float alpha = grow ? __builtin_amdgcn_exp2f(base - nb) : 1.0f;   // 0 when base is -inf
            base = nb;
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                lsum[x] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[x][db] *= alpha;
            }
        }
        const float nbase = base == -INFINITY ? 0.f : -base;
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], a.c2, nbase));
            psum += p[e];
        }
        // dense P^T: bf16 high parts and bf16 remainders, packed in pairs (a
        // bf16 P alone, even with the sums taken over the rounded weights,
        // leaves the errors of a one-sample route 1.2e-3 off)
        uint32_t hd[4], ld[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hd[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
            ld[j] = pack_bf16(p[2 * j] - __builtin_bit_cast(float, hd[j] << 16),
                              p[2 * j + 1] - __builtin_bit_cast(float, hd[j] & 0xffff0000u));
        }
        if constexpr (TWO) {
            // temporal P^T: the dense pairs outside the window zeroed (whole
            // pairs when each lane keeps all or none of its 8 keys, the usual case)
            uint32_t ht[4], lt[4];
            if (__all(bt == 0u || bt == 0xffu)) {
                const uint32_t mt = bt ? ~0u : 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ht[j] = hd[j] & mt;
                    lt[j] = ld[j] & mt;
                }
                lsum[2] += bt ? psum : 0.f;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t mt = pair_mask(bt, j);
                    ht[j] = hd[j] & mt;
                    lt[j] = ld[j] & mt;
                }
                lsum[2] = pair_sum(lt, pair_sum(ht, lsum[2]));
            }
            float dsum = psum;
            if (cross) {
                // the step where frame fa + 1 begins (once per half at most): its keys
                // of frame fa close that frame's sums, which move to the second
                // set; the first set restarts with the keys from kbnd on
                uint32_t ha[4], la[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t ma = pair_mask(bs, j);
                    ha[j] = hd[j] & ma;
                    la[j] = ld[j] & ma;
                    hd[j] &= ~ma;
                    ld[j] &= ~ma;
                }
                const bf16x8 aph = as_bf16x8(ha), apl = as_bf16x8(la);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    oacc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], aph, oacc[0][db], 0, 0, 0);
                    oacc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], apl, oacc[1][db], 0, 0, 0);
                    oacc[0][db] = f32x4{};
                }
                lsum[1] = pair_sum(la, pair_sum(ha, lsum[0]));
                lsum[0] = 0.f;
                dsum = pair_sum(ld, pair_sum(hd, 0.f));
            }
            // the step's dense P^T (from kbnd on, in the step where frame fa + 1 begins)
            lsum[0] += dsum;
            const bf16x8 dph = as_bf16x8(hd), dpl = as_bf16x8(ld), tph = as_bf16x8(ht), tpl = as_bf16x8(lt);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                oacc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], dph, oacc[0][db], 0, 0, 0);
                oacc[2][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], tph, oacc[2][db], 0, 0, 0);
                oacc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], dpl, oacc[0][db], 0, 0, 0);
                oacc[2][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], tpl, oacc[2][db], 0, 0, 0);
            }
        } else {
            lsum[0] += psum;
            // masked P^T: the dense pairs with excluded keys zeroed. Usually every lane
            // keeps all or none of its 8 keys under each mask (a range boundary falls
            // inside few of them): then whole pairs are selected
            uint32_t hs[4], ls[4], ht[4], lt[4];
            if (__all((bs == 0u || bs == 0xffu) && (bt == 0u || bt == 0xffu))) {
                const uint32_t ms = bs ? ~0u : 0u, mt = bt ? ~0u : 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hs[j] = hd[j] & ms;
                    ls[j] = ld[j] & ms;
                    ht[j] = hd[j] & mt;
                    lt[j] = ld[j] & mt;
                }
                lsum[1] += bs ? psum : 0.f;
                lsum[2] += bt ? psum : 0.f;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t ms = pair_mask(bs, j), mt = pair_mask(bt, j);
                    hs[j] = hd[j] & ms;
                    ls[j] = ld[j] & ms;
                    ht[j] = hd[j] & mt;
                    lt[j] = ld[j] & mt;
                }
                // masked sums from the masked high and low parts (their sum is p to
                // about 2^-16)
                lsum[1] = pair_sum(ls, pair_sum(hs, lsum[1]));
                lsum[2] = pair_sum(lt, pair_sum(ht, lsum[2]));
            }
            const bf16x8 ph[3] = {as_bf16x8(hd), as_bf16x8(hs), as_bf16x8(ht)};
            const bf16x8 pl[3] = {as_bf16x8(ld), as_bf16x8(ls), as_bf16x8(lt)};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int x = 0; x < 3; ++x) oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], ph[x], oacc[x][db], 0, 0, 0);
#pragma unroll
                for (int x = 0; x < 3; ++x) oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], pl[x], oacc[x][db], 0, 0, 0);
            }
        }

        // nxt holds step s+1: to LDS, then refill it with step s+AHEAD
        if (s + 1 < steps) {
            nxt.store(sm + ((s + 1) & 1) * St::STAGE, ptid);
            if (s + AHEAD < steps) nxt.load(kh, vh, kb0 + AHEAD * KSUB, N, ident, ptid);
        }
        __syncthreads();
    };
    for (int s = 0; s < steps; s += 2) {
        step(s, DEEP ? st1 : st0);
        if (s + 1 < steps) step(s + 1, st0);
    }

    if constexpr (TWO) {
        // sums of frame fa: the second set if frame fa + 1 began in the half,
        // else the first. Dense = both sets (the second is zero when unused);
        // spatial = the frames the sample's mask keeps.
        const bool crossed = c0 <= kbnd && kbnd < c0 + sub;
        const bool ka = fa < g.k || abs(fa - (int)fq) <= g.bs;
        const bool kb = fa + 1 < g.k || abs(fa + 1 - (int)fq) <= g.bs;
        const bool keep1 = crossed ? ka : false, keep0 = crossed ? kb : ka;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x4 o0 = oacc[0][db], o1 = oacc[1][db];
            oacc[0][db] = o0 + o1;
            oacc[1][db] = keep0 ? (keep1 ? o0 + o1 : o0) : (keep1 ? o1 : f32x4{});
        }
        const float l0 = lsum[0], l1 = lsum[1];
        lsum[0] = l0 + l1;
        lsum[1] = keep0 ? (keep1 ? l0 + l1 : l0) : (keep1 ? l1 : 0.f);
    }
    // ---- the two key halves of each sample block merge in LDS; half 0 writes the partial
    float lt3[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) lt3[x] = group_sum(lsum[x]);
    float* mrg = reinterpret_cast<float*>(smem) + (size_t)sb * 3 * 16 * (D + 2);   // [x][l16][D + 2]
    if (part == 1) {
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            float* w = mrg + ((size_t)x * 16 + l16) * (D + 2);
            if (grp == 0) {
                w[0] = base;
                w[1] = lt3[x];
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) w[2 + db * 16 + 4 * grp + r] = oacc[x][db][r];
        }
    }
    __syncthreads();
    if (part == 0) {
        const float b1 = mrg[(size_t)l16 * (D + 2)];
        const float m = fmaxf(base, b1);
        const float s0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(base - m);
        const float s1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(b1 - m);
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const float* w1 = mrg + ((size_t)x * 16 + l16) * (D + 2);
            float* w = a.ws + ws_index<D>(bh, chunk, a.n_chunks, x, n);
            if (grp == 0) {
                w[0] = m;
                w[1] = lt3[x] * s0 + w1[1] * s1;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = db * 16 + 4 * grp + r;
                    w[2 + d] = oacc[x][db][r] * s0 + w1[2 + d] * s1;
                }
        }
    }
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

// One thread per batch*head: sum the per-sample deviations in sample order,
// set the flag. All kMaxSamples pairs are loaded first (the workspace holds
// them for every head; slots past n_samples are never used), so the loads
// overlap instead of forming a chain.
__global__ __launch_bounds__(64) void route_flag_kernel(RArgs a, int BH) {
    const int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    const float2* e2 = reinterpret_cast<const float2*>(a.ws_err + (size_t)bh * kMaxSamples * 2);
    float2 v[kMaxSamples];
#pragma unroll
    for (int n = 0; n < kMaxSamples; ++n) v[n] = e2[n];
    float es = 0.f, et = 0.f;
#pragma unroll
    for (int n = 0; n < kMaxSamples; ++n)
        if (n < a.ns) {
            es += v[n].x;
            et += v[n].y;
        }
    a.flags[bh] = et < es ? 1 : 0;
    if (a.err) {
        a.err[2 * bh] = es;
        a.err[2 * bh + 1] = et;
    }
}

template <int D>
hipError_t launch_pair(const RArgs& r, int BH, hipStream_t stream) {
    // per-frame dense sums when a key half (chunk / 2 keys) fits in a frame
    if (r.chunk / kRouteParts <= r.g.S)
        hipLaunchKernelGGL((route_partial_kernel<D, true>), dim3(r.n_chunks, BH), dim3(kRouteBlocks * kRouteParts * 64),
                           0, stream, r);
    else
        hipLaunchKernelGGL((route_partial_kernel<D, false>), dim3(r.n_chunks, BH), dim3(kRouteBlocks * kRouteParts * 64),
                           0, stream, r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_merge_kernel<D>), dim3(r.ns, BH), dim3(D), 0, stream, r);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_flag_kernel, dim3((BH + 63) / 64), dim3(64), 0, stream, r, BH);
    return hipGetLastError();
}

}  // namespace

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
    // every call runs four 16-sample blocks (slots past n_samples repeat the last sample)
    if (a.head_dim == 64) return launch_pair<64>(r, a.BH, stream);
    return launch_pair<128>(r, a.BH, stream);
}

}  // namespace svga
