// Step 2: per-token 1x128 FP8 activation quantisation.
//
// FlashInfer PR #4287 (public-contract section) consumes activations as E4M3
// codes with one FP32 scale per token and 128-column group; its review of the
// zero-activation scale floors the scale at FLT_MIN before inversion.  The
// power-of-two scale mode follows SGLang PR #43556 (scales rounded up to
// powers of two).
//
// Layout: 16 lanes per 128-column group, each lane one 16-byte load of eight
// BF16 values (fully coalesced rows), the group amax by a 16-lane xor
// reduction, one 8-byte store of codes per lane and one scale per group.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

template <bool UE8M0>
__global__ void __launch_bounds__(256)
quant_act_kernel(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ld,
                 uint8_t *__restrict__ xq, float *__restrict__ xs) {
    quant_act_group<UE8M0>(x, M, K, ld, xq, xs, ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4,
                           threadIdx.x & 15);
}

__global__ void __launch_bounds__(256)
e4m3_encode_kernel(const float *__restrict__ in, uint8_t *__restrict__ out, int64_t n) {
    int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < 4 && i + j < n; ++j) v[j] = in[i + j];
    uint32_t w = pack_e4m3x4(v[0], v[1], v[2], v[3]);
    for (int j = 0; j < 4 && i + j < n; ++j) out[i + j] = (uint8_t)(w >> (8 * j));
}

}  // namespace

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ld,
                            uint8_t *xq, float *xs, bool ue8m0, hipStream_t st) {
    int64_t groups = M * (K >> 7);
    int64_t blocks = (groups + 15) / 16;
    if (blocks == 0) return hipSuccess;
    if (ue8m0)
        quant_act_kernel<true><<<(unsigned)blocks, 256, 0, st>>>(x, M, K, ld, xq, xs);
    else
        quant_act_kernel<false><<<(unsigned)blocks, 256, 0, st>>>(x, M, K, ld, xq, xs);
    return hipGetLastError();
}

// Counts scales that the E8M0 MFMA path cannot take as they are: anything
// but a positive power of two in [2^-126, 2^127] (sign 0, mantissa 0,
// biased exponent 1..254).  One atomic add per wave of its ballot count.
__global__ void __launch_bounds__(256)
pow2_violation_kernel(const uint32_t *__restrict__ bits, int64_t n, uint32_t *__restrict__ count) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const uint32_t b = bits[i];
        const uint32_t ex = (b >> 23) & 0xffu;
        bad += (b & 0x807fffffu) != 0u || ex == 0u || ex == 0xffu;
    }
    for (int m = 1; m < 64; m <<= 1) bad += __shfl_xor(bad, m, 64);
    if ((threadIdx.x & 63) == 0 && bad)
        __hip_atomic_fetch_add(count, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(64)
zero_word_kernel(uint32_t *p) {
    if (threadIdx.x == 0) p[0] = 0u;
}

hipError_t launch_pow2_violations(const float *scales, int64_t n, uint32_t *count, hipStream_t st) {
    zero_word_kernel<<<1, 64, 0, st>>>(count);           // a kernel, not a memset: graph-safe
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || n == 0) return err;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    pow2_violation_kernel<<<(unsigned)blocks, 256, 0, st>>>(reinterpret_cast<const uint32_t *>(scales), n,
                                                            count);
    return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float *in, uint8_t *out, int64_t n, hipStream_t st) {
    int64_t blocks = (n + 1023) / 1024;
    if (blocks == 0) return hipSuccess;
    e4m3_encode_kernel<<<(unsigned)blocks, 256, 0, st>>>(in, out, n);
    return hipGetLastError();
}

}  // namespace moe
