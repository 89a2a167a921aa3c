// Steps 3 + 4 for small grids (decode, few tokens per expert): one
// workgroup per gate/up work item of gateup_item.h (plan block, row pass,
// j-tile, K-split).
#include <type_traits>

#include "gateup_item.h"

namespace moe {

namespace {

using namespace gs;

template <int BM, int MODE>
__global__ void __launch_bounds__(512)
gateup_stream_kernel(GateUpArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int L = blockIdx.x;
    const int b = L % a.nblocks;
    L /= a.nblocks;
    const int split = L % a.nsplit;
    L /= a.nsplit;
    const int jt = L % a.jtiles;
    const int pass = L / a.jtiles;
    gateup_item<BM, MODE, 0, false>(a, smem, b, split, jt, pass, nullptr);
}

template <int BM, int MODE>
hipError_t launch_gs(const GateUpArgs &a, hipStream_t st) {
    using C = GSCfg<BM, 0, MODE == kW4>;
    const int64_t grid = (int64_t)a.nblocks * a.nsplit * a.jtiles * C::NPASS;
    if (grid == 0) return hipSuccess;
    if (a.kb_per_split < 1) return hipErrorInvalidValue;
    const int lds = C::TOTAL;
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> lds_set{0};
        const hipError_t e = raise_lds_limit(lds_set, (const void *)gateup_stream_kernel<BM, MODE>, lds);
        if (e != hipSuccess) return e;
    }
    gateup_stream_kernel<BM, MODE><<<(unsigned)grid, C::NT, lds, st>>>(a);
    return hipGetLastError();
}

template <int BM>
hipError_t launch_gs_mode(const GateUpArgs &a, int mode, hipStream_t st) {
    switch (mode) {
        case kExact: return launch_gs<BM, kExact>(a, st);
        case kFp8: return launch_gs<BM, kFp8>(a, st);
        case kFp8E8: return launch_gs<BM, kFp8E8>(a, st);
        case kExactE8: return launch_gs<BM, kExactE8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

// Route map to -1 and split-K counters to 0, in one launch.
__global__ void __launch_bounds__(256)
prep_kernel(uint32_t *__restrict__ rpos, size_t nr, uint32_t *__restrict__ cnt, size_t nc) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    for (; i < nr + nc; i += stride) {
        if (i < nr) rpos[i] = 0xffffffffu;
        else cnt[i - nr] = 0u;
    }
}

// One thread per 16-byte chunk of the packed layout (coalesced stores,
// gathered 16-byte loads): chunk q of tile (e, jt, kb) sits at tile row
// r = q / 8, position q % 8, and holds the row's chunk (q % 8) ^ (r & 7).
__global__ void __launch_bounds__(256)
prepack_w13_kernel(const uint8_t *__restrict__ w13, int64_t I, int64_t K, int64_t nchunks,
                   uint8_t *__restrict__ out) {
    const int64_t nkb = K >> 7, jtiles = I >> 7;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < nchunks;
         idx += (int64_t)gridDim.x * 256) {
        const int q = (int)(idx & 2047);
        int64_t t = idx >> 11;
        const int64_t kb = t % nkb;
        t /= nkb;
        const int64_t jt = t % jtiles, e = t / jtiles;
        const int r = q >> 3, c = (q & 7) ^ (r & 7);
        const int64_t n = (r < 128 ? jt * 128 + r : I + jt * 128 + (r - 128));
        const u32x4 v = *reinterpret_cast<const u32x4 *>(w13 + (e * 2 * I + n) * K + kb * 128 + c * 16);
        *reinterpret_cast<u32x4 *>(out + idx * 16) = v;
    }
}

}  // namespace

hipError_t launch_prepack_w13(const uint8_t *w13, int64_t E, int64_t I, int64_t K, uint8_t *out,
                              hipStream_t st) {
    const int64_t nchunks = E * 2 * I * K / 16;
    if (nchunks == 0) return hipSuccess;
    int64_t blocks = (nchunks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    prepack_w13_kernel<<<(unsigned)blocks, 256, 0, st>>>(w13, I, K, nchunks, out);
    return hipGetLastError();
}

int gateup_stream_kmax(int) { return 1 << 20; }   // the K-range streams through the ring

hipError_t launch_gateup(const GateUpArgs &a, int block_m, bool fp8_mma, bool e8m0,
                         hipStream_t st) {
    const int mode = !fp8_mma ? (e8m0 ? kExactE8 : kExact) : (e8m0 ? kFp8E8 : kFp8);
    switch (block_m) {
        case 8: return launch_gs_mode<8>(a, mode, st);
        case 16: return launch_gs_mode<16>(a, mode, st);
        case 32: return launch_gs_mode<32>(a, mode, st);
        case 64: return launch_gs_mode<64>(a, mode, st);
        case 128: return launch_gs_mode<128>(a, mode, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gateup_w4(const GateUpArgs &a, int block_m, hipStream_t st) {
    switch (block_m) {
        case 8: return launch_gs<8, kW4>(a, st);
        case 16: return launch_gs<16, kW4>(a, st);
        case 32: return launch_gs<32, kW4>(a, st);
        case 64: return launch_gs<64, kW4>(a, st);
        case 128: return launch_gs<128, kW4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prep(uint32_t *rpos, size_t n_rpos, uint32_t *cnt, size_t n_cnt, hipStream_t st) {
    const size_t n = n_rpos + n_cnt;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    prep_kernel<<<(unsigned)blocks, 256, 0, st>>>(rpos, n_rpos, cnt, n_cnt);
    return hipGetLastError();
}

}  // namespace moe
