// K / V sub-tile staging through LDS, shared by the attention and routing kernels.
//
// A sub-tile is KSUB keys x D dims of bf16. Both K and V are copied into LDS
// in their natural key-major layout (one row of D*2 bytes per key), with
// 16-byte global loads where consecutive lanes read consecutive chunks of a
// row. The MFMA A operands are then:
// * K rows for S^T = K Q^T: one 16-byte read per lane;
// * V^T rows for O^T = V^T P^T: two ds_read_b64_tr_b16 per lane. Within each
//   16-lane group that instruction hands lane 4a+b element e of source lane
//   a+4e's 8-byte read, element b. With source lane a+4e reading key k0+e,
//   dims d0+4a..d0+4a+3, lane 4a+b receives keys k0..k0+3 at dim d0+4a+b:
//   the key-contiguous operand, without any transposing store.
// Rows are padded instead of swizzled, so every operand address is one
// per-lane base plus a compile-time offset: K rows are D*2+16 bytes (an odd
// number of 16-byte units, so 16 consecutive rows read at one column hit 16
// different bank groups), V rows D*2+64 bytes (4 units past a multiple of 16,
// so the 4 keys x 4 dim-quads of one transposing read hit 16 different bank
// groups).
#pragma once

#include "svga_internal.h"

namespace svga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Bits 2 and 3 of r swapped: the key row that A-operand lane r loads.
__device__ __forceinline__ int pi32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Key index held by accumulator register i of a lane in half h of 32-key block b.
__device__ __forceinline__ int acc_key(int b, int i, int h) { return b * 32 + pi32(8 * (i >> 2) + 4 * h + (i & 3)); }

// Bits [a - kb0, b - kb0) of a 64-bit mask over keys kb0 .. kb0+63 (clamped).
__device__ __forceinline__ uint64_t window_bits(int a, int b, int kb0) {
    const int lo = imin(imax(a - kb0, 0), 64), hi = imin(imax(b - kb0, 0), 64);
    const uint64_t below_hi = hi >= 64 ? ~0ull : (1ull << hi) - 1;
    const uint64_t below_lo = lo >= 64 ? ~0ull : (1ull << lo) - 1;
    return below_hi & ~below_lo;
}

// Raw buffer resource over bytes bytes from p (no stride, gfx9 data format):
// buffer loads at offsets at or past bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// VPAD: V row padding in bytes (64 suits a_v's lane layout; other read
// patterns pick their own).
template <int D, int KSUB, int NT, int VPAD = 64>
struct Stager {
    static constexpr int RV = D / 8;                 // 16-byte chunks per row
    static constexpr int CH = KSUB * RV;             // chunks per tensor per sub-tile
    static constexpr int CU = (CH + NT - 1) / NT;    // chunks per thread per tensor
    static constexpr int KROW = D * 2 + 16;          // padded K row (bytes)
    static constexpr int VROW = D * 2 + VPAD;        // padded V row (bytes)
    static constexpr int KBYTES = KSUB * KROW;
    static constexpr int STAGE = KBYTES + KSUB * VROW;   // K tile, then V tile

    uint4 kreg[CU];
    uint4 vreg[CU];

    __device__ __forceinline__ static int k_off(int row, int chunk) { return row * KROW + chunk * 16; }
    __device__ __forceinline__ static int v_off(int row, int chunk) { return KBYTES + row * VROW + chunk * 16; }

    // Load keys kb0 .. kb0+KSUB-1 (rows >= limit read as zero). src(j) maps a
    // key index to the row actually read.
    template <class Src>
    __device__ __forceinline__ void load(const uint16_t* kh, const uint16_t* vh, int kb0, int limit, Src src, int tid) {
#pragma unroll
        for (int r = 0; r < CU; ++r) {
            const int u = tid + r * NT;
            if (CH % NT == 0 || u < CH) {
                const int row = u / RV, c = u % RV;
                const int j = kb0 + row;
                if (j < limit) {
                    const size_t off = (size_t)src(j) * D;
                    kreg[r] = reinterpret_cast<const uint4*>(kh + off)[c];
                    vreg[r] = reinterpret_cast<const uint4*>(vh + off)[c];
                } else {
                    kreg[r] = uint4{0, 0, 0, 0};
                    vreg[r] = uint4{0, 0, 0, 0};
                }
            }
        }
    }

    // Byte offset in the K / V buffers of chunk r of thread tid for source row
    // j; j < 0 gives an offset beyond the buffer's end, which buffer loads
    // read as zero (no branch around the load).
    __device__ __forceinline__ static int chunk_off(int r, int tid, int j) {
        const int c = (tid + r * NT) % RV;
        return j >= 0 ? j * (D * 2) + c * 16 : 0x7ffffff0;
    }
    // Chunk r of load() at a byte offset found by chunk_off.
    __device__ __forceinline__ void load_chunk_off(int r, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int off) {
        kreg[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
        vreg[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
    // Chunk r of store() from the thread's chunk-0 addresses kl = stage +
    // k_off(row0, c), vl = stage + v_off(row0, c): chunk r is NT / RV rows on.
    __device__ __forceinline__ void store_chunk_at(int r, char* kl, char* vl) const {
        static_assert(NT % RV == 0, "chunks of one thread share a column");
        *reinterpret_cast<uint4*>(kl + r * (NT / RV) * KROW) = kreg[r];
        *reinterpret_cast<uint4*>(vl + r * (NT / RV) * VROW) = vreg[r];
    }

    // Row of the sub-tile that chunk r of thread tid holds.
    __device__ __forceinline__ static int chunk_row(int r, int tid) { return (tid + r * NT) / RV; }

    __device__ __forceinline__ void store(char* stage, int tid) const {
#pragma unroll
        for (int r = 0; r < CU; ++r) {
            const int u = tid + r * NT;
            if (CH % NT == 0 || u < CH) {
                const int row = u / RV, c = u % RV;
                *reinterpret_cast<uint4*>(stage + k_off(row, c)) = kreg[r];
                *reinterpret_cast<uint4*>(stage + v_off(row, c)) = vreg[r];
            }
        }
    }

    // A operand of S^T = K Q^T: key row b*32 + pi32(l32), dims 16c + 8h .. +7.
    __device__ __forceinline__ static bf16x8 a_k(const char* stage, int b, int c, int l32, int h) {
        return *reinterpret_cast<const bf16x8*>(stage + k_off(b * 32 + pi32(l32), 2 * c + h));
    }

    // Per-lane part of the V^T operand address (see a_v).
    __device__ __forceinline__ static int v_lane_off(int lane) {
        const int g = lane >> 4, j = lane & 15, qa = j & 3, e = j >> 2;
        return ((g >> 1) * 8 + e) * VROW + ((g & 1) * 2 + (qa >> 1)) * 16 + (qa & 1) * 8;
    }

    // A operand of O^T = V^T P^T: dim row db*32 + (lane % 32), keys 16 m16 + 8h .. +7
    // (h = lane / 32), from two transposing reads of four keys each. Source
    // lane 16g + 4e + qa reads key 16 m16 + 8(g/2) + e (+4 for the second
    // read), dims db*32 + 16(g%2) + 4qa .. +3.
    __device__ __forceinline__ static bf16x8 a_v(const char* stage, int db, int m16, int vlane_off) {
        const char* p0 = stage + KBYTES + vlane_off + m16 * 16 * VROW + db * 64;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * VROW));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, both);
    }
};

}  // namespace svga
