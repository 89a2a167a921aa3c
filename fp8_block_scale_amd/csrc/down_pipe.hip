// Step 5 for large grids: the down-projection GEMM as a persistent kernel
// with a three-stage LDS pipeline fed by direct global->LDS loads.
//
// Same arithmetic as down.hip (FlashInfer PR #4287, PR summary and the FP32
// scale note of its final kernel performance section): for plan row p of
// expert e holding route r,
//   y[r, c] = w_r * sum_jb h_s[p, jb] * w2_s[e, c / 128, jb]
//                         * sum_{j in jb} h_q[p, j] * W2[e, c, j]     (FP32)
// written to the route-indexed buffer y[r, :] (the finalize kernel adds a
// token's routes in route order).
//
// Work items are (row tile, 256 output columns); the row tiles are the ones
// the gate/up prep kernel listed in the workspace (up to 128 consecutive plan
// rows of one expert).  One workgroup (8 waves) per CU pulls items from the
// per-XCD counters (all column tiles of a row tile on one XCD, so the
// tile's intermediate rows are fetched into its L2 once).  Per 128-deep step of the intermediate dimension a stage
// holds the W2 tile (256 rows x 128 B), the tile's intermediate rows
// (128 x 128 B, contiguous in plan order) and their scales; rows are
// XOR-swizzled in LDS as in the gate/up pipeline.  FP8 MFMA
// (v_mfma_f32_16x16x128_f8f6f4) with the FP32 scale product applied per step,
// or with power-of-two scales as E8M0 exponents inside the MFMA.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRows = 128;
constexpr int kNT = 512;
constexpr int kStages = 3;
constexpr int kWBytes = 256 * 128;
constexpr int kHBytes = kRows * 128;
constexpr int kWInstr = kWBytes / 1024 / 8;
constexpr int kHInstr = kHBytes / 1024 / 8;
constexpr int kPerStage = kWInstr + kHInstr + 1;
constexpr int kMaxJb = 256;                   // I <= 32768

__device__ __forceinline__ v8i join8q(const u32x4 &lo, const u32x4 &hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

template <int BM, bool E8M0>
__global__ void __launch_bounds__(kNT, 1)
down_pipe_kernel(DownArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *sW = smem;                                            // [kStages][256][128]
    uint8_t *sH = smem + kStages * kWBytes;                        // [kStages][128][128]
    float *sHs = reinterpret_cast<float *>(sH + kStages * kHBytes); // [kStages][128]
    float *sSw = sHs + kStages * kRows;                            // [2][kMaxJb] w2_s blocks
    int *sRt = reinterpret_cast<int *>(sSw + 2 * kMaxJb);          // [128] route or -1
    int *sItem = sRt + kRows;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = w & 3, wm = w >> 2;
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t I = a.I, K = a.K;
    const int njb = a.njb;
    const int ntiles = a.tmeta[0];
    const int home = blockIdx.x & 7;
    int q = 0;                                       // position in the XCD ranges (thread 0)

    for (;;) {
        if (tid == 0) sItem[0] = next_xcd_item(a.tmeta + 9, ntiles, a.ctiles, home, q);
        __syncthreads();
        const int item = sItem[0];
        if (item < 0) break;
        // a row tile's column tiles are consecutive items on one XCD
        const int ct = item % a.ctiles;
        const int2 tl = a.tiles[item / a.ctiles];
        const int b = tl.x, nb = tl.y;
        const int e = a.eids[b];
        if (e < 0 || e >= a.E) {
            __syncthreads();
            continue;
        }
        const int nrows = nb * BM;
        const int64_t p0 = (int64_t)b * BM;
        const int64_t c0 = (int64_t)ct * 256;
        const int ncols = K - c0 < 256 ? (int)(K - c0) : 256;     // 128 or 256

        if (tid < kRows) {
            int r = -1;
            if (tid < nrows) {
                int v = a.sorted[p0 + tid];
                if (v >= 0 && (int64_t)v < a.R) r = v;
            }
            sRt[tid] = r;
        }
        {
            // the two 128-column scale blocks of this column tile
            const float *s0 = a.w2s + ((int64_t)e * (K >> 7) + (c0 >> 7)) * njb;
            for (int i = tid; i < njb; i += kNT) {
                sSw[i] = s0[i];
                sSw[kMaxJb + i] = ncols > 128 ? s0[njb + i] : 0.f;
            }
        }
        __syncthreads();

        // DMA sources of this lane
        const int sub = lane >> 3, slot = lane & 7;
        const uint8_t *wsrc[kWInstr];
#pragma unroll
        for (int i = 0; i < kWInstr; ++i) {
            const int row = (w * kWInstr + i) * 8 + sub;              // 0..255
            const int64_t c = c0 + (row < ncols ? row : 0);
            wsrc[i] = a.w2 + ((int64_t)e * K + c) * I + (slot ^ (row & 7)) * 16;
        }
        const uint8_t *hsrc[kHInstr];
#pragma unroll
        for (int i = 0; i < kHInstr; ++i) {
            const int row = (w * kHInstr + i) * 8 + sub;
            const int64_t p = p0 + (row < nrows ? row : 0);
            hsrc[i] = a.hq + p * I + (slot ^ (row & 7)) * 16;
        }
        const float *ssrc;
        {
            const int row = w * 16 + (lane & 15);
            ssrc = a.hs + (p0 + (row < nrows ? row : 0)) * njb;
        }
        auto issue = [&](int stage, int jb) {
            uint8_t *dw = sW + stage * kWBytes + (w * kWInstr) * 1024;
#pragma unroll
            for (int i = 0; i < kWInstr; ++i)
                __builtin_amdgcn_global_load_lds(wsrc[i] + (int64_t)jb * 128, dw + i * 1024, 16, 0, 0);
            uint8_t *dh = sH + stage * kHBytes + (w * kHInstr) * 1024;
#pragma unroll
            for (int i = 0; i < kHInstr; ++i)
                __builtin_amdgcn_global_load_lds(hsrc[i] + (int64_t)jb * 128, dh + i * 1024, 16, 0, 0);
            if (lane < 16)
                __builtin_amdgcn_global_load_lds(ssrc + jb, sHs + stage * kRows + w * 16, 4, 0, 0);
        };

        constexpr int NU = 4;
        const bool wave_on = (wm * 64 < nrows) && (64 * wn < ncols);
        v4f acc[4][NU];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int u = 0; u < NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};

        // One pipeline step: wait for stage ST (step jb), refill stage
        // (ST + 2) % 3 with step jb + 2, multiply.  The stage indices are
        // compile-time constants so the compiler can tell the refilled and
        // the read LDS ranges apart and keeps the refill in flight.
        auto step = [&](auto st_c, int jb) {
            constexpr int ST = decltype(st_c)::value;
            if (jb + 2 < njb) {
                issue((ST + 2) % kStages, jb + 2);
                wait_vmcnt<2 * kPerStage>();
            } else if (jb + 1 < njb) {
                wait_vmcnt<kPerStage>();
            } else {
                wait_vmcnt<0>();
            }
            stage_barrier();
            if (wave_on) {
                // this wave's 64 columns lie in one 128-column scale block
                const float sb = sSw[(wn >= 2 ? kMaxJb : 0) + jb];
                const uint8_t *Ws = sW + ST * kWBytes;
                const uint8_t *Hs = sH + ST * kHBytes;
                const float *Ss = sHs + ST * kRows;
                v8i wq[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int row = 64 * wn + 16 * s + l16;
                    const uint8_t *rp = Ws + row * 128;
                    const u32x4 lo = lds_read16(rp + ((g ^ (row & 7)) * 16));
                    const u32x4 hi = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                    wq[s] = join8q(lo, hi);
                }
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    if (wm * 64 + u * 16 >= nrows) continue;
                    const int row = wm * 64 + u * 16 + l16;
                    const uint8_t *rp = Hs + row * 128;
                    const u32x4 lo = lds_read16(rp + ((g ^ (row & 7)) * 16));
                    const u32x4 hi = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                    const v8i B = join8q(lo, hi);
                    const float sa = Ss[row];
                    if constexpr (E8M0) {
                        const int ea = e8m0_of(sb), eb = e8m0_of(sa);
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc[s][u] = mfma16x16x128_e8m0(wq[s], B, acc[s][u], ea, eb);
                    } else {
                        const float f = sa * sb;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            v4f t = mfma16x16x128(wq[s], B);
                            acc[s][u] = t * f + acc[s][u];
                        }
                    }
                }
            }
            stage_barrier();
        };
        issue(0, 0);
        if (njb > 1) issue(1, 1);
        for (int jb = 0; jb < njb; jb += kStages) {
            step(std::integral_constant<int, 0>{}, jb);
            if (jb + 1 < njb) step(std::integral_constant<int, 1>{}, jb + 1);
            if (jb + 2 < njb) step(std::integral_constant<int, 2>{}, jb + 2);
        }

        if (wave_on) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int row = wm * 64 + u * 16 + l16;
                const int r = sRt[row];
                if (r < 0) continue;
                const float wr = a.topk_w[r];
                float *dst = a.y + (int64_t)r * K + c0 + 64 * wn + 4 * g;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    *reinterpret_cast<v4f *>(dst + 16 * s) = acc[s][u] * wr;
            }
        }
        __syncthreads();
    }
}

constexpr size_t kSmem = (size_t)kStages * (kWBytes + kHBytes) + kStages * kRows * 4 +
                         2 * kMaxJb * 4 + kRows * 4 + 16;

int num_cus_dn() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int BM, bool E8M0>
hipError_t launch_dn_pipe(const DownArgs &a, hipStream_t st) {
    if (a.nblocks == 0) return hipSuccess;
    int64_t grid = num_cus_dn();
    const int64_t max_items = (int64_t)a.nblocks * a.ctiles;
    if (grid > max_items) grid = max_items;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void *)down_pipe_kernel<BM, E8M0>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmem);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    down_pipe_kernel<BM, E8M0><<<(unsigned)grid, kNT, kSmem, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_down_pipe(const DownArgs &a, int block_m, bool e8m0, hipStream_t st) {
    switch (block_m) {
        case 16: return e8m0 ? launch_dn_pipe<16, true>(a, st) : launch_dn_pipe<16, false>(a, st);
        case 32: return e8m0 ? launch_dn_pipe<32, true>(a, st) : launch_dn_pipe<32, false>(a, st);
        case 64: return e8m0 ? launch_dn_pipe<64, true>(a, st) : launch_dn_pipe<64, false>(a, st);
        case 128: return e8m0 ? launch_dn_pipe<128, true>(a, st) : launch_dn_pipe<128, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
