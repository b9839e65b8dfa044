// Token permutation between frame-major (F, H, W) and the temporal order
// (ASTA section "Arrange tokens for efficient temporal access", Figure 9),
// applied per head from a device flag with fixed tensor shapes (ASTA section
// "Support dynamic routing with fixed tensor shapes").
//
// Both directions are written as gathers: every output row is written once,
// in order, with 16-byte non-temporal stores (streamed past the caches: 6.9
// against 5.4 TB/s with ordinary stores); each input row (head_dim * 2 bytes,
// 256 B at head_dim 128) is read whole by consecutive lanes. HBM-bound: one
// read and one write of the tensor.
#include "svga_internal.h"

namespace svga {

namespace {

typedef unsigned u32x4nt __attribute__((ext_vector_type(4)));   // for the non-temporal store builtin
constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte vectors per thread, loaded before any store

__global__ __launch_bounds__(kThreads) void permute_kernel(const uint4* __restrict__ in, uint4* __restrict__ out,
                                                           const uint8_t* __restrict__ flags, Geo g,
                                                           FastDiv div_vecs, int32_t row_vecs, int inverse) {
    const int32_t bh = blockIdx.y;
    const bool temporal = flags[bh] != 0;
    const int64_t head_vecs = (int64_t)g.N * row_vecs;
    const uint4* src = in + (int64_t)bh * head_vecs;
    uint4* dst = out + (int64_t)bh * head_vecs;
    const uint32_t base = (uint32_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    const uint32_t hv = (uint32_t)head_vecs;
    auto fetch = [&](uint32_t e) {
        uint32_t r, c;
        div_vecs.divmod(e, r, c);
        int32_t sr = (int32_t)r;
        if (temporal) sr = inverse ? temporal_dst(g, sr) : temporal_src(g, sr);
        return src[(int64_t)sr * row_vecs + c];
    };
    uint4 v[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const uint32_t e = base + i * kThreads;
        v[i] = e < hv ? fetch(e) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const uint32_t e = base + i * kThreads;
        if (e < hv) __builtin_nontemporal_store(__builtin_bit_cast(u32x4nt, v[i]), reinterpret_cast<u32x4nt*>(dst + e));
    }
}

}  // namespace

hipError_t launch_permute(const void* in, void* out, const uint8_t* flags, int32_t BH, const Geo& g, int32_t head_dim,
                          bool inverse, hipStream_t stream) {
    const int32_t row_vecs = head_dim / 8;
    const int64_t head_vecs = (int64_t)g.N * row_vecs;   // below 2^31: checked by the caller
    FastDiv dv((uint32_t)row_vecs);
    dim3 grid((unsigned)((head_vecs + kThreads * kUnroll - 1) / (kThreads * kUnroll)), (unsigned)BH);
    hipLaunchKernelGGL(permute_kernel, grid, dim3(kThreads), 0, stream, static_cast<const uint4*>(in),
                       static_cast<uint4*>(out), flags, g, dv, row_vecs, inverse ? 1 : 0);
    return hipGetLastError();
}

}  // namespace svga
