// K / V sub-tile staging through LDS, shared by the attention and routing kernels.
//
// A sub-tile is KSUB keys x D dims of bf16. K is stored key-major (one row of
// D*2 bytes per key), V transposed to dim-major (one row of KSUB*2 bytes per
// dim), so that both MFMA A operands (K rows for S^T = K Q^T, V^T rows for
// O^T = V^T P^T) are single 16-byte LDS reads. 16-byte chunks are XOR-swizzled
// so that the 16 lanes of each read quarter-wave touch distinct bank groups.
// Global loads are 16 bytes per lane; consecutive lanes read consecutive
// chunks of one key row, so every row is read whole.
#pragma once

#include "svga_internal.h"

namespace svga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Bits 2 and 3 of r swapped: the key row that A-operand lane r loads.
__device__ __forceinline__ int pi32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int D, int KSUB, int NT>
struct Stager {
    static constexpr int RV = D / 8;                 // 16-byte vectors per row
    static constexpr int KCH = KSUB * RV;            // K chunks per sub-tile
    static constexpr int KU = (KCH + NT - 1) / NT;
    static constexpr int VUN = (KSUB / 4) * RV;      // V units: 4 keys x 8 dims
    static constexpr int VU = (VUN + NT - 1) / NT;
    static constexpr int KBYTES = KSUB * D * 2;
    static constexpr int STAGE = 2 * KBYTES;         // K tile, then V^T tile

    uint4 kreg[KU];
    uint4 vreg[VU][4];

    __device__ __forceinline__ static int k_off(int row, int chunk) {
        int swz;
        if constexpr (D == 128) swz = pi32(row & 15);
        else swz = (pi32(row & 31) >> 1) & 7;
        return row * (D * 2) + ((chunk ^ swz) << 4);
    }
    __device__ __forceinline__ static int v_off(int d, int chunk) {
        int swz;
        if constexpr (KSUB == 64) swz = (d >> 1) & 7;
        else swz = (d >> 2) & 3;
        return KBYTES + d * (KSUB * 2) + ((chunk ^ swz) << 4);
    }

    // Load keys kb0 .. kb0+KSUB-1 (rows >= limit read as zero). src(j) maps a
    // key index to the row actually read.
    template <class Src>
    __device__ __forceinline__ void load(const uint16_t* kh, const uint16_t* vh, int kb0, int limit, Src src, int tid) {
#pragma unroll
        for (int r = 0; r < KU; ++r) {
            const int u = tid + r * NT;
            if (KCH % NT == 0 || u < KCH) {
                const int row = u / RV, c = u % RV;
                const int j = kb0 + row;
                kreg[r] = j < limit ? reinterpret_cast<const uint4*>(kh + (size_t)src(j) * D)[c] : uint4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int r = 0; r < VU; ++r) {
            const int u = tid + r * NT;
            if (VUN % NT == 0 || u < VUN) {
                const int dg = u % RV, kq = u / RV;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = kb0 + 4 * kq + e;
                    vreg[r][e] = j < limit ? reinterpret_cast<const uint4*>(vh + (size_t)src(j) * D)[dg] : uint4{0, 0, 0, 0};
                }
            }
        }
    }

    __device__ __forceinline__ void store(char* stage, int tid) const {
#pragma unroll
        for (int r = 0; r < KU; ++r) {
            const int u = tid + r * NT;
            if (KCH % NT == 0 || u < KCH) {
                const int row = u / RV, c = u % RV;
                *reinterpret_cast<uint4*>(stage + k_off(row, c)) = kreg[r];
            }
        }
#pragma unroll
        for (int r = 0; r < VU; ++r) {
            const int u = tid + r * NT;
            if (VUN % NT == 0 || u < VUN) {
                const int dg = u % RV, kq = u / RV;
                const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vreg[r][0]);
                const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vreg[r][1]);
                const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vreg[r][2]);
                const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vreg[r][3]);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    // dims 8dg+2x (low halves) and 8dg+2x+1 (high halves) of keys 4kq..4kq+3
                    uint2 lo, hi;
                    lo.x = (r0[x] & 0xffffu) | (r1[x] << 16);
                    lo.y = (r2[x] & 0xffffu) | (r3[x] << 16);
                    hi.x = (r0[x] >> 16) | (r1[x] & 0xffff0000u);
                    hi.y = (r2[x] >> 16) | (r3[x] & 0xffff0000u);
                    const int d0 = 8 * dg + 2 * x;
                    *reinterpret_cast<uint2*>(stage + v_off(d0, kq >> 1) + (kq & 1) * 8) = lo;
                    *reinterpret_cast<uint2*>(stage + v_off(d0 + 1, kq >> 1) + (kq & 1) * 8) = hi;
                }
            }
        }
    }

    // A operand of S^T = K Q^T: key row b*32 + pi32(l32), dims 16c + 8h .. +7.
    __device__ __forceinline__ static bf16x8 a_k(const char* stage, int b, int c, int l32, int h) {
        return *reinterpret_cast<const bf16x8*>(stage + k_off(b * 32 + pi32(l32), 2 * c + h));
    }
    // A operand of O^T = V^T P^T: dim row db*32 + l32, keys 16 m16 + 8h .. +7.
    __device__ __forceinline__ static bf16x8 a_v(const char* stage, int db, int m16, int l32, int h) {
        return *reinterpret_cast<const bf16x8*>(stage + v_off(db * 32 + l32, 2 * m16 + h));
    }
};

// Key index held by accumulator register i of a lane in half h of 32-key block b.
__device__ __forceinline__ int acc_key(int b, int i, int h) { return b * 32 + pi32(8 * (i >> 2) + 4 * h + (i & 3)); }

}  // namespace svga
