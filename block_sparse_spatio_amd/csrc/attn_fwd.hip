// Block-sparse flash-attention forward for gfx950 (MI355X), bf16 in, fp32 accumulate.
//
// ASTA section "Logical sparsity is not physical sparsity": attention is
// computed tile by tile, Q[i1:i2] K[j1:j2]^T, with softmax statistics carried
// across tiles, and excluded pairs set to minus infinity inside visited
// tiles. Section "Avoid intra-tile masking when there is nothing to mask":
// full tiles take a path with no mask at all, boundary tiles the masked path,
// both feeding the same running statistics. Section "Align the sparse mask
// with final execution": positions past the sequence end get zero weight.
//
// Design (one workgroup per (batch*head, query tile)):
// * WAVES waves, each owning QB blocks of 32 query rows. Q stays in VGPRs as
//   the B operand of v_mfma_f32_32x32x16_bf16 for the whole kernel. With
//   QB = 1 and 8 waves a workgroup holds two waves per SIMD and each wave
//   stays within 256 registers, so one wave's softmax (VALU) runs while the
//   other wave's matrix products occupy the MFMA pipe.
// * Scores are computed transposed, S^T = K Q^T (A = K rows from LDS), so each
//   lane holds one query's scores: row max and row sum are lane-local plus one
//   exchange with the other 32-lane half.
// * The A-operand lane r loads key row pi(r) (bits 2 and 3 of r swapped). With
//   the 32x32 accumulator layout (register i of lane l is row 8(i/4)+4(l/32)+i%4)
//   this puts keys 16m+8h..16m+8h+7 in registers 8m..8m+7 of half h, which is
//   exactly the B-operand layout that P^T needs for O^T = V^T P^T.
// * K and V sub-tiles of KSUB keys are copied to LDS through registers, with
//   the global loads for step s+2 in flight while step s computes; V^T
//   operands come from transposing LDS reads; rows are padded so that all
//   operand reads are conflict-free (tile_stage.h).
// * Ping-pong (8-wave workgroups): waves w and w+4 share a SIMD. Each step
//   has two phases with one workgroup barrier between them; in one phase a
//   wave issues only matrix products (PV of the previous step, then Q K^T of
//   this step), in the other only the softmax of this step's scores. Waves
//   0-3 run the phases in one order and waves 4-7 in the other, so on every
//   SIMD one wave's products overlap the other wave's softmax. Only waves 4-7
//   move K and V: in their softmax phase they store the next step's staged
//   registers and load the step after, one chunk between blocks of
//   exponentials, so the products of waves 0-3 never wait behind load issue;
//   the barrier after that phase publishes the stage. Smaller workgroups
//   have no partner wave: they run QK^T, softmax and PV in turn. 512-row
//   query tiles run as two 256-row workgroups.
// * Lazy rescaling: a row keeps its exponent base until its running max
//   exceeds the base by more than 2^8 in probability scale; only then are the
//   output accumulator and the row sum rescaled. The final normalisation uses
//   the same base, so the result is the plain softmax.
// * FULL tiles run a loop with no mask code at all; BOUNDARY tiles run a
//   second loop that applies the exact mask (NAIVE / EXACT maps) or the
//   padding mask (DENSE / ROUNDED maps). A row with no kept key so far keeps
//   an exponent base of zero, so no NaN appears.
// * Persistent launch (with a workspace): one workgroup per resident slot
//   takes work items from a global counter. With the split-tail workspace
//   the last items (one per resident 8-wave workgroup) run as kSplitParts
//   pieces over contiguous shares of their key tile lists, each piece writing
//   its normalised output and log-sum-exp, and merge_kernel combines them;
//   the end of the launch then waits on a quarter of an item, not a whole one.
// * Workgroups keep the hardware's round-robin spread over the 8 XCDs:
//   every XCD gets every eighth query tile of every head, so the XCDs carry
//   equal work. (Grouping consecutive query tiles on one XCD for L2 reuse
//   measured slower: the XCDs' shares of work then differ and the last XCD
//   sets the end, while K/V re-reads are cheap at this arithmetic intensity.)
#include <atomic>
#include <type_traits>

#include "tile_stage.h"

namespace svga {

namespace {

struct KArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const uint8_t* flags;
    const int32_t* n_full;  // [2][tq]
    const int32_t* n_bnd;   // [2][tq]
    const int32_t* kv;      // [2][tq][tk]
    Geo g;
    int32_t tq, tk, bkv;
    int32_t exact;          // 1: exact mask on boundary tiles, 0: padding only
    int32_t qparts;         // workgroups per map query tile (its rows split in parts of this kernel's BQ)
    int32_t total;          // work items: BH * tq * qparts
    int32_t* counter;       // persistent mode: next work unit (zeroed before the launch); else null
    // Persistent mode with a split tail: items first_split .. total-1 run as
    // kSplitParts pieces each, piece p taking the p-th contiguous share of the
    // item's key tiles. Work units: the whole items below first_split, then
    // the pieces, item by item.
    int32_t units;          // first_split + (total - first_split) * kSplitParts
    int32_t first_split;    // total when no item is split
    int32_t split;          // 1: the workspace holds the split-tail region
    float* part_lse;        // [kSplitItemsMax * kSplitParts][BQ] log-sum-exp of each piece's rows
    uint16_t* part_o;       // [kSplitItemsMax * kSplitParts][BQ][D] normalised output of each piece (bf16)
    float c2;               // softmax_scale * log2(e)
    float scale;
};

constexpr float kRescaleLog2 = 8.0f;   // rescale when the running max grows by more than 2^8

// max of x over the two 32-lane halves, in every lane: v_permlane32_swap
// exchanges the halves of its two operands, so one of the two results holds
// the other half's value whatever the lane.
__device__ __forceinline__ float half_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(fmaxf(x, __builtin_bit_cast(float, (uint32_t)r[0])), __builtin_bit_cast(float, (uint32_t)r[1]));
}

template <int D, int QB>
struct WaveState {
    static constexpr int DB = D / 32;
    f32x16 oacc[QB][DB];
    float base[QB];   // exponent base of the row (log2 domain, scale folded in)
    float lsum[QB];   // per-lane partial row sum (this half's keys)
};

// The pieces of one step of KSUB keys for one wave.
template <int D, int QB, int KSUB, int NT>
struct Step {
    using St = Stager<D, KSUB, NT>;
    static constexpr int KBLK = KSUB / 32;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    typedef f32x16 Scores[QB][KBLK];
    typedef bf16x8 Probs[QB][KSUB / 16];

    // S^T = K Q^T for the keys staged at stg (compiler-scheduled).
    static __device__ __forceinline__ void qk(const char* stg, const bf16x8 (&qreg)[QB][DC], Scores& sacc, int lane) {
        const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int b = 0; b < KBLK; ++b) sacc[qb][b] = f32x16{};
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int b = 0; b < KBLK; ++b) {
                const bf16x8 ak = St::a_k(stg, b, c, l32, h);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[qb][c], sacc[qb][b], 0, 0, 0);
            }
    }

    // O^T += V^T P^T for the values staged at stg (compiler-scheduled).
    static __device__ __forceinline__ void pv(const char* stg, const Probs& preg, WaveState<D, QB>& ws, int lane) {
        const int vlo = St::v_lane_off(lane);
#pragma unroll
        for (int m16 = 0; m16 < KSUB / 16; ++m16)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 av = St::a_v(stg, db, m16, vlo);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    ws.oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, preg[qb][m16], ws.oacc[qb][db], 0, 0, 0);
            }
    }

    // Matrix phase of the ping-pong: PV of the previous step (DO_PV, values at
    // vstg), then S^T = K Q^T of this step (DO_QK, keys at kstg). One product
    // per slot, each slot's operand read issued LA slots ahead, the order
    // fixed with sched_barrier so that the products issue back to back and
    // the operand registers in flight stay bounded.
    template <bool DO_PV, bool DO_QK>
    static __device__ __forceinline__ void products(const char* vstg, const char* kstg, const Probs& preg,
                                                    const bf16x8 (&qreg)[QB][DC], Scores& sacc,
                                                    WaveState<D, QB>& ws, int lane) {
        constexpr int NPV = DO_PV ? (KSUB / 16) * DB : 0;
        constexpr int NS = NPV + (DO_QK ? KBLK * DC : 0);
        constexpr int LA = 6;
        const int l32 = lane & 31, h = lane >> 5;
        const int vlo = St::v_lane_off(lane);
        // slot j < NPV: PV product (m16 = j / DB, db = j % DB); slot NPV + i:
        // score product (c = i / KBLK, b = i % KBLK)
        auto operand = [&](int j) __attribute__((always_inline)) {
            if (j < NPV) return St::a_v(vstg, j % DB, j / DB, vlo);
            const int i = j - NPV;
            return St::a_k(kstg, i % KBLK, i / KBLK, l32, h);
        };
        if constexpr (DO_QK) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int b = 0; b < KBLK; ++b) sacc[qb][b] = f32x16{};
        }
        bf16x8 op[NS];
#pragma unroll
        for (int j = 0; j < LA && j < NS; ++j) op[j] = operand(j);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (j + LA < NS) op[j + LA] = operand(j + LA);
            if (j < NPV) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    ws.oacc[qb][j % DB] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[j], preg[qb][j / DB], ws.oacc[qb][j % DB], 0, 0, 0);
            } else {
                const int i = j - NPV;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[qb][i % KBLK] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[j], qreg[qb][i / KBLK], sacc[qb][i % KBLK], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Mask (MASKED only), row max with lazy rescaling, P = exp2(S c2 - base)
    // rounded to bf16 for the PV products, fp32 row sums. hook(k), k = 0 ..
    // 2 KBLK - 1, is called after each block of 8 exponentials: code placed
    // there (with its own sched_barriers) is spread over the phase.
    template <bool MASKED, class Hook>
    static __device__ __forceinline__ void softmax(Scores& sacc, Probs& preg, WaveState<D, QB>& ws,
                                                   const RowKeys (&rk)[QB], const KArgs& a, int kb0, int lane,
                                                   Hook hook) {
        const int h = lane >> 5;
        if constexpr (MASKED) {
            bool periodic = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) periodic = periodic || (a.exact && rk[qb].periodic);
            if (__any(periodic)) {
                // sink frames of the literal temporal order: an element-wise test
#pragma unroll
                for (int b = 0; b < KBLK; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int j = kb0 + acc_key(b, i, h);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) {
                            const bool keep = a.exact ? row_keeps(a.g, rk[qb], j) : (j < a.g.N);
                            if (!keep) sacc[qb][b][i] = -INFINITY;
                        }
                    }
            } else {
                // the row keeps at most two key ranges: a 64-bit keep mask over the
                // step's keys, shifted so that bit acc_key(b, i, 0) belongs to this
                // lane's element (b, i); then a bit test and a select per element
                // (a bitwise-select form of the same test is miscompiled by the
                // gfx950 backend's three-input bit-op combine, so it is not used)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    uint64_t m = a.exact ? window_bits(rk[qb].a0, rk[qb].b0, kb0) | window_bits(rk[qb].a1, rk[qb].b1, kb0)
                                         : window_bits(0, a.g.N, kb0);
                    m >>= acc_key(0, 0, h);   // 8 for the upper half-wave, 0 for the lower
                    const uint32_t mw[2] = {(uint32_t)m, (uint32_t)(m >> 32)};
#pragma unroll
                    for (int b = 0; b < KBLK; ++b)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int pos = acc_key(b, i, 0) - 32 * b;
                            if (!((mw[b] >> pos) & 1u)) sacc[qb][b][i] = -INFINITY;
                        }
                }
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = sacc[qb][0][0];
#pragma unroll
            for (int b = 0; b < KBLK; ++b)
#pragma unroll
                for (int i = (b == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, sacc[qb][b][i]);
            mx = half_max(mx);
            // a new base is needed when this step's max exceeds the current base by more than 2^8
            const float cand = mx * a.c2;
            const bool grow = cand > ws.base[qb] + kRescaleLog2;
            if (__any(grow)) {
                const float nb = grow ? cand : ws.base[qb];
                // rows that keep their base scale by 1 (their base may still be -inf);
                // a growing row whose old base is -inf scales its zero state by 0
                const float alpha = grow ? __builtin_amdgcn_exp2f(ws.base[qb] - nb) : 1.0f;
                ws.base[qb] = nb;
                ws.lsum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) ws.oacc[qb][db] *= alpha;
            }
            const float nbase = ws.base[qb] == -INFINITY ? 0.f : -ws.base[qb];
            float ls = 0.f;
#pragma unroll
            for (int b = 0; b < KBLK; ++b) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int i = 8 * m; i < 8 * m + 8; ++i) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[qb][b][i], a.c2, nbase));
                        sacc[qb][b][i] = p;
                        ls += p;
                    }
                    bf16x8 pk;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pk[e] = (__bf16)sacc[qb][b][8 * m + e];
                    preg[qb][2 * b + m] = pk;
                    if (qb == 0) hook(2 * b + m);
                }
            }
            ws.lsum[qb] += ls;
        }
    }

    // The values a phase hands to the next one must be computed before the
    // barrier between them: these empty asm statements use them there, so no
    // instruction that produces them sinks into the following phase.
    static __device__ __forceinline__ void fence(const Scores& sacc) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int b = 0; b < KBLK; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(sacc[qb][b][i]));
    }
    static __device__ __forceinline__ void fence(const Probs& preg, const WaveState<D, QB>& ws) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int m = 0; m < KSUB / 16; ++m) asm volatile("" ::"v"(preg[qb][m]));
            asm volatile("" ::"v"(ws.lsum[qb]), "v"(ws.base[qb]));
        }
    }
};

// The one workgroup barrier of a ping-pong step, between its two phases: it
// waits for this wave's LDS writes (the stage that waves 4-7 stored in the
// phase before it becomes visible), and sched_barrier keeps the scheduler from
// moving work across it.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// Four bf16 (round to nearest even) to p[0..3].
__device__ __forceinline__ void store_bf16x4(uint16_t* p, float x0, float x1, float x2, float x3) {
    uint2 w;
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x2) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x3) << 16);
    *reinterpret_cast<uint2*>(p) = w;
}

// QB = 1: at most 256 registers per wave, so two waves share each SIMD (two
// 4-wave workgroups, or one 8-wave workgroup, per CU).
// One work item: the rows of (batch*head, query tile, part) `logical`. With
// slot >= 0 the item is split: piece slot % kSplitParts of its key tiles
// only, its state kept in piece slot `slot` (split item slot / kSplitParts).
template <int D, int QB, int WAVES, int KSUB, bool GATHER>
__device__ __forceinline__ void attn_item(const KArgs& a, const int logical, const int slot, char* smem) {
    constexpr bool PINGPONG = WAVES == 8 && QB == 1;
    constexpr int NT = WAVES * 64;
    constexpr int BQ = WAVES * QB * 32;
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    using St = Stager<D, KSUB, NT>;
    using Sp = Step<D, QB, KSUB, NT>;
    if (logical >= a.total) return;
    const int per_bh = a.tq * a.qparts;
    const int bh = logical / per_bh;
    const int qrem = logical - bh * per_bh;
    const int qt = qrem / a.qparts;                                   // query tile of the map
    const int row0 = qt * BQ * a.qparts + (qrem - qt * a.qparts) * BQ;   // first row of this part
    const int N = a.g.N;
    const int kind = a.flags[bh] ? SVGA_KIND_TEMPORAL : SVGA_KIND_SPATIAL;
    const bool gat = GATHER && kind == SVGA_KIND_TEMPORAL;
    // The tile list is read-only for the whole kernel; reading it through the
    // constant address space lets the compiler use scalar loads for it even
    // after barriers and LDS stores (a vector load there would put a full
    // memory latency in front of every step's K / V loads).
    typedef const __attribute__((address_space(4))) int32_t* ConstI32;
    ConstI32 kvl = (ConstI32)(a.kv + ((size_t)kind * a.tq + qt) * a.tk);
    // list lengths and key-tile ids come from device memory: clamp them so
    // that no map content can send a load outside the K / V tensors
    int nf = imin(imax(a.n_full[kind * a.tq + qt], 0), a.tk);
    int ntiles = imin(nf + imax(a.n_bnd[kind * a.tq + qt], 0), a.tk);
    // Only the 8-wave ping-pong kernels run split items (kSplitWaves); in the
    // others the piece code would cost the main loop registers.
    constexpr bool SPLITS = WAVES == kSplitWaves && QB == 1;
    if (SPLITS && slot >= 0) {
        // a piece: the key tiles t0 .. t1-1 of the list
        constexpr int P = (int)kSplitParts;
        const int part = slot - (slot / P) * P;
        const int t0 = ntiles * part / P, t1 = ntiles * (part + 1) / P;
        kvl += t0;
        nf = imin(imax(nf - t0, 0), t1 - t0);
        ntiles = t1 - t0;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const size_t head_off = (size_t)bh * N * D;
    const uint16_t* qh = a.q + head_off;
    const uint16_t* kh = a.k + head_off;
    const uint16_t* vh = a.v + head_off;
    const Geo& g = a.g;

    // ---- Q rows of this lane, as B operands (d = 16c + 8h .. +7)
    bf16x8 qreg[QB][DC];
    RowKeys rk[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = row0 + (wave * QB + qb) * 32 + l32;
        if (row < N) {
            const int qsrc = gat ? temporal_src(g, row) : row;
            const bf16x8* p = reinterpret_cast<const bf16x8*>(qh + (size_t)qsrc * D + 8 * h);
#pragma unroll
            for (int c = 0; c < DC; ++c) qreg[qb][c] = p[2 * c];
        } else {
#pragma unroll
            for (int c = 0; c < DC; ++c) qreg[qb][c] = bf16x8{};
        }
        rk[qb] = row_keys(g, kind, row < N ? row : N - 1);
    }

    WaveState<D, QB> ws;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        ws.base[qb] = -INFINITY;
        ws.lsum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) ws.oacc[qb][db] = f32x16{};
    }

    const int nsub = a.bkv / KSUB;
    const int steps = ntiles * nsub;
    St st;
    auto src = [&](int j) { return GATHER ? (gat ? temporal_src(g, j) : j) : j; };
    auto key_base = [&](int s) {
        const int t = s / nsub;
        return imin(imax(kvl[t], 0), a.tk - 1) * a.bkv + (s - t * nsub) * KSUB;
    };

    const int sfull = nf * nsub;
    typename Sp::Scores sacc;
    typename Sp::Probs preg;
    if constexpr (!PINGPONG) {
        if (steps > 0) {
            st.load(kh, vh, key_base(0), N, src, tid);
            st.store(smem, tid);
            if (steps > 1) st.load(kh, vh, key_base(1), N, src, tid);
        }
        __syncthreads();
        // full tiles first (no mask code at all), then boundary tiles; both
        // loops carry the same state and the same double-buffered pipeline
        auto advance = [&](int s) {
            if (s + 1 < steps) {
                st.store(smem + ((s + 1) & 1) * St::STAGE, tid);
                if (s + 2 < steps) st.load(kh, vh, key_base(s + 2), N, src, tid);
            }
            __syncthreads();
        };
        int s = 0;
        for (; s < sfull; ++s) {
            const char* stg = smem + (s & 1) * St::STAGE;
            Sp::qk(stg, qreg, sacc, lane);
            Sp::template softmax<false>(sacc, preg, ws, rk, a, 0, lane, [](int) {});
            Sp::pv(stg, preg, ws, lane);
            advance(s);
        }
        for (; s < steps; ++s) {
            const char* stg = smem + (s & 1) * St::STAGE;
            Sp::qk(stg, qreg, sacc, lane);
            Sp::template softmax<true>(sacc, preg, ws, rk, a, key_base(s), lane, [](int) {});
            Sp::pv(stg, preg, ws, lane);
            advance(s);
        }
    } else {
        // K / V staging: ring of four LDS stages, filled through the registers
        // of waves 4-7 only. In its vector phase of step s each of those waves
        // stores step s+1's registers to stage s+1 and loads step s+2's, one
        // chunk at a time between the blocks of exponentials, so that neither
        // the LDS writes nor the load issue form a burst; waves 0-3 issue no
        // memory traffic in the loop. Step s's products read stages s-1 (V)
        // and s (K); stage s+1 was last read in step s-2, before the barrier
        // of step s-1, so the four stages never overlap a write with a read,
        // and the barrier in the middle of step s publishes stage s+1 to the
        // products of step s+1. That one barrier per step also keeps the two
        // wave groups half a step apart; a second one at the step top (tried)
        // only added its wait. Loads past the last step repeat its keys (never
        // stored where anyone reads).
        auto stage = [&](int s) { return (const char*)(smem + (s & 3) * St::STAGE); };
        auto wstage = [&](int s) { return smem + (s & 3) * St::STAGE; };
        const bool lead = wave < WAVES / 2;   // products first
        using Sh = Stager<D, KSUB, NT / 2>;
        Sh sh;
        const int htid = tid - NT / 2;
        const __amdgpu_buffer_rsrc_t rsk = head_rsrc(kh, N * D * 2);
        const __amdgpu_buffer_rsrc_t rsv = head_rsrc(vh, N * D * 2);
        auto next_keys = [&](int s) __attribute__((always_inline)) { return key_base(imin(s + 2, steps - 1)); };
        if (steps > 0 && !lead) {
            sh.load(kh, vh, key_base(0), N, src, htid);
            sh.store(wstage(0), htid);
            sh.load(kh, vh, key_base(imin(1, steps - 1)), N, src, htid);
        }
        // step top: a barrier only before the first step (stage 0 from the
        // prologue), otherwise a scheduling fence
        auto first_top = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        auto top = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
        // buffer offsets of the rows that step s's transfer loads, found in the
        // matrix phase before it (where VALU time is free), so that the vector
        // phase only issues the loads; gathered rows: lane i finds the source
        // of key kb + i and each chunk takes its row's from that lane. The LDS
        // side stores at one per-thread base per tensor plus constant offsets.
        int loff[Sh::CU];
        auto prep = [&](int s) __attribute__((always_inline)) {
            if constexpr (GATHER) {
                const int my = next_keys(s) + lane;
                const int mysrc = lane < KSUB && my < N ? (gat ? temporal_src(g, my) : my) : -1;
#pragma unroll
                for (int r = 0; r < Sh::CU; ++r) loff[r] = Sh::chunk_off(r, htid, __shfl(mysrc, Sh::chunk_row(r, htid)));
            } else {
                const int kb = next_keys(s);
#pragma unroll
                for (int r = 0; r < Sh::CU; ++r) {
                    const int j = kb + Sh::chunk_row(r, htid);
                    loff[r] = Sh::chunk_off(r, htid, j < N ? j : -1);
                }
            }
        };
        const int kl0 = Sh::k_off(htid / Sh::RV, htid % Sh::RV), vl0 = Sh::v_off(htid / Sh::RV, htid % Sh::RV);
        // softmax of step t; with XFER (waves 4-7, step s) the stage transfer rides along
        auto soft = [&](auto masked, auto xfer, int t, int s) __attribute__((always_inline)) {
            char* dst = wstage(s + 1);

            // chunk r goes with hook point r * NH / CU (NH = KSUB / 16 points)
            auto hook = [&](int k) __attribute__((always_inline)) {
                if constexpr (decltype(xfer)::value) {
                    constexpr int NH = KSUB / 16;
#pragma unroll
                    for (int r = 0; r < Sh::CU; ++r) {
                        if (r * NH / Sh::CU != k) continue;
                        __builtin_amdgcn_sched_barrier(0);
                        sh.store_chunk_at(r, dst + kl0, dst + vl0);
                        sh.load_chunk_off(r, rsk, rsv, loff[r]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            };
            if constexpr (decltype(masked)::value)
                Sp::template softmax<true>(sacc, preg, ws, rk, a, key_base(t), lane, hook);
            else
                Sp::template softmax<false>(sacc, preg, ws, rk, a, 0, lane, hook);
            Sp::fence(preg, ws);
        };
        // products of step s: PV of step s-1 (if any) and QK^T of step s (if any),
        // issued at raised wave priority so that the SIMD's arbiter prefers the
        // matrix wave over its partner's vector work
        auto prod = [&](auto both, int s) __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(1);
            if constexpr (decltype(both)::value)
                Sp::template products<true, true>(stage(s - 1), stage(s), preg, qreg, sacc, ws, lane);
            else if (s == 0)
                Sp::template products<false, true>(nullptr, stage(0), preg, qreg, sacc, ws, lane);
            else
                Sp::template products<true, false>(stage(s - 1), nullptr, preg, qreg, sacc, ws, lane);
            Sp::fence(sacc);
            __builtin_amdgcn_s_setprio(0);
        };
        using Both = std::true_type;
        using One = std::false_type;
        using Yes = std::true_type;
        using No = std::false_type;
        // Every wave passes the same steps + 2 barriers. The first and last
        // steps are peeled so that the loops hold one form of each phase.
        const int sf = imin(sfull, steps);
        if (steps == 0) {
            __syncthreads();
            phase_barrier();
        } else if (lead) {
            first_top();
            prod(One{}, 0);
            phase_barrier();
            if (0 < sfull) soft(No{}, No{}, 0, 0);
            else soft(Yes{}, No{}, 0, 0);
            int s = 1;
            for (; s < sf; ++s) {
                top();
                prod(Both{}, s);
                phase_barrier();
                soft(No{}, No{}, s, s);
            }
            for (; s < steps; ++s) {
                top();
                prod(Both{}, s);
                phase_barrier();
                soft(Yes{}, No{}, s, s);
            }
            top();
            prod(One{}, steps);
            phase_barrier();
        } else {
            first_top();
            sh.store(wstage(1), htid);
            sh.load(kh, vh, next_keys(0), N, src, htid);
            phase_barrier();
            prod(One{}, 0);
            prep(1);
            int s = 1;
            for (; s < imin(sf + 1, steps); ++s) {
                top();
                soft(No{}, Yes{}, s - 1, s);
                phase_barrier();
                prod(Both{}, s);
                prep(s + 1);
            }
            for (; s < steps; ++s) {
                top();
                soft(Yes{}, Yes{}, s - 1, s);
                phase_barrier();
                prod(Both{}, s);
                prep(s + 1);
            }
            top();
            if (steps - 1 < sfull) soft(No{}, No{}, steps - 1, steps);
            else soft(Yes{}, No{}, steps - 1, steps);
            phase_barrier();
            prod(One{}, steps);
        }
    }

    // ---- epilogue: O = acc / l, bf16 round-to-nearest-even; LSE = (base + log2 l) * ln 2.
    // A piece of a split item writes both to its slot (rows relative to the
    // item, LSE always) for merge_kernel.
    const bool piece = SPLITS && slot >= 0;
    constexpr int BQROWS = WAVES * QB * 32;
    uint16_t* obase = piece ? a.part_o + (size_t)slot * BQROWS * D
                            : a.o + head_off;
    float* lbase = piece ? a.part_lse + (size_t)slot * BQROWS
                         : (a.lse ? a.lse + (size_t)bh * N : nullptr);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = ws.lsum[qb] + __shfl_xor(ws.lsum[qb], 32);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int row = row0 + (wave * QB + qb) * 32 + l32;
        if (row < N) {
            const int orow = piece ? row - row0 : (gat ? temporal_src(g, row) : row);
            uint16_t* op = obase + (size_t)orow * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    store_bf16x4(op + db * 32 + 8 * gq + 4 * h, ws.oacc[qb][db][4 * gq] * inv,
                                 ws.oacc[qb][db][4 * gq + 1] * inv, ws.oacc[qb][db][4 * gq + 2] * inv,
                                 ws.oacc[qb][db][4 * gq + 3] * inv);
            }
            if (lbase && h == 0)
                lbase[orow] = lt > 0.f ? (ws.base[qb] + __log2f(lt)) * 0.6931471805599453f : -INFINITY;
        }
    }
}

// Without a counter, one workgroup per work item in index order. With one,
// persistent workgroups (one per CU) take the next item from the counter until
// none is left: no workgroup launch between items, and a free CU takes work at
// once instead of waiting while the in-order dispatcher blocks on a full XCD.
template <int D, int QB, int WAVES, int KSUB, bool GATHER>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(QB == 1 ? 2 : 1)))
void attn_fwd_kernel(KArgs a) {
    constexpr bool PINGPONG = WAVES == 8 && QB == 1;
    using St = Stager<D, KSUB, WAVES * 64>;
    __shared__ __attribute__((aligned(16))) char smem[(PINGPONG ? 4 : 2) * St::STAGE];
    __shared__ int next;
    if (!a.counter) {
        attn_item<D, QB, WAVES, KSUB, GATHER>(a, blockIdx.x, -1, smem);
        return;
    }
    for (;;) {
        if (threadIdx.x == 0) next = atomicAdd(a.counter, 1);
        __syncthreads();
        const int t = next;
        __syncthreads();   // every wave has read `next` before it changes; the last item's LDS reads are done
        if (t >= a.units) break;
        if constexpr (WAVES == kSplitWaves && QB == 1) {
            // unit u past first_split is piece slot u: item first_split + u / kSplitParts
            const int slot = t >= a.first_split ? t - a.first_split : -1;
            const int logical = slot >= 0 ? a.first_split + slot / (int)kSplitParts : t;
            attn_item<D, QB, WAVES, KSUB, GATHER>(a, logical, slot, smem);
        } else {
            attn_item<D, QB, WAVES, KSUB, GATHER>(a, t, -1, smem);   // no split items here
        }
    }
}

__global__ void zero_counter_kernel(int32_t* c) {
    if (threadIdx.x == 0) *c = 0;
}

// Merge of the split items' pieces (ASTA section "Avoid intra-tile masking
// when there is nothing to mask": partial results over disjoint key sets
// combine through their softmax statistics). Piece p of a row holds its
// normalised output O_p and log-sum-exp L_p; with m = max_p L_p and
// w_p = e^(L_p - m): O = sum_p w_p O_p / sum_p w_p, LSE = m + ln sum_p w_p.
// A piece that kept no key of the row has L_p = -inf and weight 0. One
// thread per 8 dims of one row; `rows` = query rows of one work item.
template <int D, bool GATHER>
__global__ __launch_bounds__(256) void merge_kernel(KArgs a, int rows) {
    constexpr int CH = D / 8;
    constexpr int P = (int)kSplitParts;
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int item = gid / (rows * CH);
    if (item >= a.total - a.first_split) return;
    const int rem = gid - item * rows * CH;
    const int r = rem / CH, c = rem - r * CH;
    const int logical = a.first_split + item;
    const int N = a.g.N;
    const int per_bh = a.tq * a.qparts;
    const int bh = logical / per_bh;
    const int qrem = logical - bh * per_bh;
    const int qt = qrem / a.qparts;
    const int row = qt * rows * a.qparts + (qrem - qt * a.qparts) * rows + r;
    if (row >= N) return;
    const size_t slot0 = (size_t)item * P;
    const float* part_lse = a.part_lse;
    const uint16_t* part_o = a.part_o;
    float lp[P];
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        lp[p] = part_lse[(slot0 + p) * rows + r];
        m = fmaxf(m, lp[p]);
    }
    float w[P];
    float wsum = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        w[p] = lp[p] > -INFINITY ? __builtin_amdgcn_exp2f((lp[p] - m) * 1.4426950408889634f) : 0.f;
        wsum += w[p];
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint4 x = *reinterpret_cast<const uint4*>(part_o + ((slot0 + p) * rows + r) * D + 8 * c);
        const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w[p] * __builtin_bit_cast(float, u[e] << 16);
            acc[2 * e + 1] += w[p] * __builtin_bit_cast(float, u[e] & 0xffff0000u);
        }
    }
    const int orow = GATHER && a.flags[bh] ? temporal_src(a.g, row) : row;
    uint16_t* op = a.o + ((size_t)bh * N + orow) * D + 8 * c;
    store_bf16x4(op, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    store_bf16x4(op + 4, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    if (a.lse && c == 0) a.lse[(size_t)bh * N + orow] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

// Workgroups of one kernel instance that the current device holds at once
// (CUs x occupancy), queried once per (instance, device) and cached: the
// attribute and occupancy queries cost host time that every call would pay.
constexpr int kMaxDevices = 64;
template <int D, int QB, int WAVES, int KSUB, bool GATHER>
hipError_t resident_workgroups(int* out) {
    static std::atomic<int> cache[kMaxDevices];   // 0: not queried yet
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return hipSuccess;
        }
    }
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_kernel<D, QB, WAVES, KSUB, GATHER>,
                                                         WAVES * 64, 0);
    if (e != hipSuccess) return e;
    const int r = imax(cus, 1) * imax(per_cu, 1);
    if (cached) cache[dev].store(r, std::memory_order_relaxed);
    *out = r;
    return hipSuccess;
}

template <int D, int QB, int WAVES, int KSUB>
hipError_t launch_one(const KArgs& k0, bool gather, hipStream_t stream) {
    KArgs k = k0;
    k.units = k.total;
    k.first_split = k.total;
    unsigned nwg = (unsigned)k.total;
    if (k.counter) {
        // as many workgroups as can be resident at once
        int resident = 0;
        const hipError_t e = gather ? resident_workgroups<D, QB, WAVES, KSUB, true>(&resident)
                                    : resident_workgroups<D, QB, WAVES, KSUB, false>(&resident);
        if (e != hipSuccess) return e;
        // split tail: the last min(resident, total) items (at most the
        // workspace's capacity) run in pieces
        const int nsplit = k.split && WAVES == kSplitWaves && QB == 1 ? imin(imin(resident, k.total), (int)kSplitItemsMax) : 0;
        k.first_split = k.total - nsplit;
        k.units = k.first_split + nsplit * (int)kSplitParts;
        nwg = (unsigned)imin(k.units, resident);
        hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(64), 0, stream, k.counter);
    }
    if (nwg == 0) return hipGetLastError();
    dim3 grid(nwg);
    if (gather)
        hipLaunchKernelGGL((attn_fwd_kernel<D, QB, WAVES, KSUB, true>), grid, dim3(WAVES * 64), 0, stream, k);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, QB, WAVES, KSUB, false>), grid, dim3(WAVES * 64), 0, stream, k);
    const int nsplit = k.total - k.first_split;
    if (nsplit > 0) {
        constexpr int ROWS = WAVES * QB * 32;
        const unsigned threads = (unsigned)nsplit * ROWS * (D / 8);
        const dim3 mgrid((threads + 255) / 256);
        if (gather)
            hipLaunchKernelGGL((merge_kernel<D, true>), mgrid, dim3(256), 0, stream, k, ROWS);
        else
            hipLaunchKernelGGL((merge_kernel<D, false>), mgrid, dim3(256), 0, stream, k, ROWS);
    }
    return hipGetLastError();
}

// bq -> (QB, WAVES): 32 -> (1,1), 64 -> (1,2), 128 -> (1,4), 256 -> (1,8); a 512-row
// query tile runs as two 256-row workgroups that walk the same tile lists (64-row
// waves do not fit two per SIMD without spilling).
// KSUB = 64 when bkv is a multiple of 64, else 32.
template <int D>
hipError_t dispatch(const KArgs& k, int bq, int ksub, bool gather, hipStream_t stream, bool* sup) {
    *sup = true;
    if (ksub == 64) {
        if (bq == 32) return launch_one<D, 1, 1, 64>(k, gather, stream);
        if (bq == 64) return launch_one<D, 1, 2, 64>(k, gather, stream);
        if (bq == 128) return launch_one<D, 1, 4, 64>(k, gather, stream);
        if (bq == 256) return launch_one<D, 1, 8, 64>(k, gather, stream);
        if (bq == 512) {
            // two 256-row parts per 512-row query tile, each walking that tile's lists
            KArgs k2 = k;
            k2.qparts = 2;
            k2.total = k.total * 2;
            return launch_one<D, 1, 8, 64>(k2, gather, stream);
        }
    } else {
        if (bq == 32) return launch_one<D, 1, 1, 32>(k, gather, stream);
        if (bq == 64) return launch_one<D, 1, 2, 32>(k, gather, stream);
        if (bq == 128) return launch_one<D, 1, 4, 32>(k, gather, stream);
        if (bq == 256) return launch_one<D, 1, 8, 32>(k, gather, stream);
        if (bq == 512) {
            KArgs k2 = k;
            k2.qparts = 2;
            k2.total = k.total * 2;
            return launch_one<D, 1, 8, 32>(k2, gather, stream);
        }
    }
    *sup = false;
    return hipSuccess;
}

}  // namespace

hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t stream, bool* supported) {
    *supported = attn_supported(a.head_dim, a.bq, a.bkv);
    if (!*supported) return hipSuccess;
    KArgs k;
    k.q = static_cast<const uint16_t*>(a.q);
    k.k = static_cast<const uint16_t*>(a.k);
    k.v = static_cast<const uint16_t*>(a.v);
    k.o = static_cast<uint16_t*>(a.o);
    k.lse = a.lse;
    k.flags = a.flags;
    k.n_full = reinterpret_cast<const int32_t*>(a.map + a.L.n_full);
    k.n_bnd = reinterpret_cast<const int32_t*>(a.map + a.L.n_bnd);
    k.kv = reinterpret_cast<const int32_t*>(a.map + a.L.kv);
    k.g = a.geo;
    k.tq = a.L.tq;
    k.tk = a.L.tk;
    k.bkv = a.bkv;
    k.exact = (a.mode == SVGA_MAP_NAIVE || a.mode == SVGA_MAP_EXACT) ? 1 : 0;
    k.qparts = 1;
    k.total = a.BH * a.L.tq;
    k.counter = a.counter;
    k.split = a.counter && a.split ? 1 : 0;
    k.part_lse = nullptr;
    k.part_o = nullptr;
    if (k.split) {
        char* base = reinterpret_cast<char*>(a.counter);
        k.part_lse = reinterpret_cast<float*>(base + kSplitLseOffset);
        k.part_o = reinterpret_cast<uint16_t*>(base + kSplitLseOffset + split_lse_bytes(a.bq));
    }
    k.c2 = a.scale * 1.4426950408889634f;
    k.scale = a.scale;
    const int ksub = a.bkv % 64 == 0 ? 64 : 32;
    if (a.head_dim == 64) return dispatch<64>(k, a.bq, ksub, a.gather != 0, stream, supported);
    return dispatch<128>(k, a.bq, ksub, a.gather != 0, stream, supported);
}

}  // namespace svga
