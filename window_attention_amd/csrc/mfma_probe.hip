// win_probe_mfma_loop: the chip's sustained bf16 MFMA rate on changing
// register data, a measurement beside the attention path (bench.py's
// practical ceilings), not part of it.
//
// Every wave runs eight independent accumulation chains of
// v_mfma_f32_32x32x16_bf16.  The A and B operands are four fragments each,
// loaded once per lane from the caller's buffer (for example N(0,1) bf16
// values) and rotated between the MFMAs of a chain, so the matrix cores see
// changing data with no memory traffic inside the loop.  Under the chip's
// power limit the rate depends on the data: zero operands run at the full
// clock, random ones do not.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;
constexpr int kThreads = 256;

// iters is a multiple of 4: the operand rotation repeats every 4 MFMAs of a
// chain, which keeps every register index a compile-time constant.
__global__ __launch_bounds__(kThreads, 2) void mfma_loop_kernel(const bf16x8* __restrict__ src, int64_t frags,
                                                                float* __restrict__ out, int32_t iters) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = src[(t * 8 + i) % frags];
        b[i] = src[(t * 8 + 4 + i) % frags];
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int32_t it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[(c + u) & 3], acc[c], 0, 0, 0);
    }
    // one value per lane keeps every chain live
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[t] = s;
}

}  // namespace

// src: device bf16 [src_elems], src_elems a positive multiple of 8 (16-byte
// aligned); out: device fp32 [blocks * 256]; iters: MFMAs per chain, rounded
// up to a multiple of 4.  Useful work per call: blocks * 4 waves * 8 chains *
// iters * 32768 flops.  Returns 0, -1 (bad argument) or -4 (HIP error).
extern "C" int win_probe_mfma_loop(const void* src, int64_t src_elems, float* out, int32_t blocks, int32_t iters,
                                   void* stream) {
    if (!src || !out || src_elems < 8 || src_elems % 8 || blocks <= 0 || iters <= 0) return -1;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(out) & 3u)) return -1;
    const int32_t it4 = iters > (INT32_MAX - 3) ? INT32_MAX - 3 : iters;
    mfma_loop_kernel<<<dim3((uint32_t)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const bf16x8*>(src), src_elems / 8, out, (it4 + 3) / 4 * 4);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
