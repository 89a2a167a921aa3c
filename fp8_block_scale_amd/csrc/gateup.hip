// Steps 3 + 4 for small grids (decode, few tokens per expert): gate/up
// grouped GEMM with 128x128 FP32 weight block scales, SwiGLU, and FP8
// requantisation of the SwiGLU output per plan row and 128-column group.
//
// What is computed (FlashInfer PR #4287, PR summary and public-contract
// section): for plan row p of block b (expert e = expert_ids[b], route
// r = sorted[p], token t = r / top_k)
//   g[p, n] = sum_kb x_s[t, kb] * w13_s[e, n / 128, kb]
//                    * sum_{k in kb} x_q[t, k] * W13[e, n, k]        (FP32)
//   h[p, j] = silu(g[p, j]) * g[p, I + j],  silu(v) = v / (1 + e^-v)
//   h_q[p, j], h_s[p, j / 128] = FP8 group quantisation of h (FP32 or
//   power-of-two scale rule; the FLT_MIN floor keeps all-zero rows finite).
//
// Here the weights are the whole cost: a block holds one or two valid rows,
// so the kernel is a weight stream.  One workgroup = one plan block (its
// valid rows, in passes of at most 64) x one 128-wide intermediate tile
// (128 gate rows + 128 up rows of W13) x one K-range; eight waves take 16
// gate and the matching 16 up rows each.  Every wave streams its 32 weight
// rows straight into registers, four 128-byte K-blocks per row per stage
// (512 contiguous bytes of each row, which keeps HBM pages open), with two
// stages in flight and no barrier in the loop.  The activation rows and all
// scales of the K-range are gathered into LDS once, up front.
//
// The MMA is the 16x16 tile with weights as the A operand (16 rows) and
// tokens as B (16 columns); lane (l % 16, l / 16) ends with four consecutive
// rows of one token.  Three MMA modes:
//   kExact  (default) E4M3 codes widened exactly to FP16 in registers and
//           multiplied with v_mfma_f32_16x16x32_f16 (exact products, FP32
//           accumulation);
//   kFp8    v_mfma_f32_16x16x128_f8f6f4 on the codes directly;
//   kFp8E8  as kFp8 with power-of-two scales applied inside the MFMA.
//
// K is split over workgroups; each writes the partial sums of its valid rows
// to the workspace and the last one of a tile to arrive (atomic counter)
// adds them in split order -- deterministic -- and finishes the tile.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

enum { kExact = 0, kFp8 = 1, kFp8E8 = 2 };

template <int BM>
struct GSCfg {
    static constexpr int RP = BM < 64 ? BM : 64;   // plan rows per pass
    static constexpr int NPASS = BM / RP;
    static constexpr int NU = RP / 16;             // 16-token subtiles
    static constexpr int NT = 512;                 // eight waves
    static constexpr int S = 4;                    // K-blocks per stage
    static constexpr int LPS = 4 * S;              // 16-byte loads per stage per lane
    static constexpr int KMAX = 1024 / RP;         // K-blocks per workgroup (128 KB x tile)
    static constexpr int GROW = 260;               // row stride of the FP32 tile
};

// LDS carve-up, shared by the kernel and its launcher: the activation tile
// (RP rows of KMAX K-blocks, 16-byte chunks XOR-swizzled by row & 7 within
// each K-block), reused after the K loop as the FP32 tile [RP][GROW]; the
// activation scales [RP][KMAX]; the weight scales [2][KMAX]; routes; flags.
template <int BM>
struct GSLayout {
    using C = GSCfg<BM>;
    static constexpr int XROWB = C::KMAX * 128;
    static constexpr int X0 = C::RP * XROWB, G0 = C::RP * C::GROW * 4;
    static constexpr int XS = X0 > G0 ? X0 : G0;
    static constexpr int WS = XS + C::RP * C::KMAX * 4;
    static constexpr int TOK = WS + 2 * C::KMAX * 4;
    static constexpr int XT = TOK + C::RP * 4;
    static constexpr int MISC = XT + C::RP * 4;
    static constexpr int TOTAL = MISC + 16;
};

template <int BM, int MODE>
__global__ void __launch_bounds__(512)
gateup_stream_kernel(GateUpArgs a) {
    using C = GSCfg<BM>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using Ld = GSLayout<BM>;
    const int kps = a.kb_per_split;
    uint8_t *sX = smem;
    float *sG = reinterpret_cast<float *>(smem);    // reuses the x tile after the loop
    float *sXs = reinterpret_cast<float *>(smem + Ld::XS);
    float *sWs = reinterpret_cast<float *>(smem + Ld::WS);
    int *sTok = reinterpret_cast<int *>(smem + Ld::TOK);   // route of each row, -1 if none
    int *sXt = reinterpret_cast<int *>(smem + Ld::XT);     // token whose x row fills the row
    int *sMisc = reinterpret_cast<int *>(smem + Ld::MISC);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    int L = blockIdx.x;
    const int b = L % a.nblocks;
    L /= a.nblocks;
    const int split = L % a.nsplit;
    L /= a.nsplit;
    const int jt = L % a.jtiles;
    const int pass = L / a.jtiles;
    const int row0 = pass * C::RP;

    // the plan entries of this pass are read together with the block's
    // expert (every entry below sorted_cap is readable)
    int r = -1;
    if (w == 0 && lane < C::RP) r = a.sorted[(int64_t)b * BM + row0 + lane];
    const int ntp = a.ntp[0];
    const int e = __builtin_amdgcn_readfirstlane(a.eids[b]);   // uniform: scalar descriptors
    if (b * BM >= ntp || e < 0 || e >= a.E) return;   // padded block

    for (int i = tid; i < C::RP * C::KMAX; i += C::NT) sXs[i] = 0.f;
    // this pass's routes (wave 0), the valid-row extent, the inverse plan map
    if (w == 0) {
        if (lane < C::RP) {
            r = (r >= 0 && (int64_t)r < a.R) ? r : -1;
            sTok[lane] = r;
            if (r >= 0 && jt == 0 && split == 0) a.rpos[r] = b * BM + row0 + lane;
        }
        const uint64_t m = __ballot(r >= 0);
        const int nv = m ? 64 - __builtin_clzll(m) : 0;
        const int t = r >= 0 ? r / a.top_k : -1;
        const int tlast = __shfl(t, nv > 0 ? nv - 1 : 0, 64);
        if (lane < C::RP) sXt[lane] = t >= 0 ? t : tlast;
        if (lane == 0) sMisc[0] = nv;
    }
    __syncthreads();
    const int nvp = sMisc[0];                   // rows [0, nvp) hold every valid row
    if (nvp == 0) return;                       // whole pass masked (same for all splits)

    const int kb0 = split * kps;
    const int kb1 = kb0 + kps < a.nkb ? kb0 + kps : a.nkb;
    const int nk = kb1 - kb0;
    const int nst = (nk + C::S - 1) / C::S;
    const int64_t K = a.K, I = a.I;

    // ---- weight stream: this wave's 16 gate rows and the matching up rows,
    // through buffer descriptors over the tile's 128 gate / 128 up rows.
    // Stages past the K-range read at an offset beyond the descriptor, which
    // returns zeros without touching memory: every stage issues the same
    // loads, so the loop has no branches and the waits stay exact.
    const uint8_t *gbase = a.w13 + ((int64_t)e * 2 * I + (int64_t)jt * 128) * K;
    const __amdgpu_buffer_rsrc_t rg =
        __builtin_amdgcn_make_buffer_rsrc((void *)gbase, (short)0, (int)(128 * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t ru =
        __builtin_amdgcn_make_buffer_rsrc((void *)(gbase + I * K), (short)0, (int)(128 * K), 0x00020000);
    const int rowoff = (16 * w + l16) * (int)K + 16 * g;
    const int past = (int)(128 * K);            // first offset past the descriptor
    u32x4 wb[2][C::S][4];
    auto issue = [&](int st, auto BUF) {
        constexpr int bf = decltype(BUF)::value;
        const int vo = st < nst ? rowoff + (kb0 + st * C::S) * 128 : past;
#pragma unroll
        for (int kk = 0; kk < C::S; ++kk) {
            wb[bf][kk][0] = __builtin_amdgcn_raw_buffer_load_b128(rg, vo + kk * 128, 0, 0);
            wb[bf][kk][1] = __builtin_amdgcn_raw_buffer_load_b128(rg, vo + kk * 128 + 64, 0, 0);
            wb[bf][kk][2] = __builtin_amdgcn_raw_buffer_load_b128(ru, vo + kk * 128, 0, 0);
            wb[bf][kk][3] = __builtin_amdgcn_raw_buffer_load_b128(ru, vo + kk * 128 + 64, 0, 0);
        }
    };
    // ---- activation rows [0, nvpad) of the K-range (LDS DMA: lane l of an
    // instruction fills 16-byte slot l of a 1 KB run of one row), their
    // scales, the weight scales.  Masked and padding rows read the last
    // valid row's token (sXt); their columns are never stored.
    const int nvpad = (nvp + 15) & ~15;
    {
        constexpr int SPR = C::KMAX * 8;        // slots per row
        constexpr int NI = C::RP * SPR / 64;    // DMA instructions for a full tile
        const int tv = sXt[lane < C::RP ? lane : 0];   // row tokens, one per lane
#pragma unroll
        for (int i = 0; i < NI / 8; ++i) {
            const int q = i * 8 + w;
            const int row = q * 64 / SPR, slot0 = q * 64 % SPR;
            if (row < nvpad && slot0 < nk * 8) {
                const int t = __builtin_amdgcn_readlane(tv, row);
                const int c = (slot0 + lane) ^ (row & 7);
                const int kbl = (c >> 3) < nk ? (c >> 3) : 0;
                lds_dma16(a.xq + (int64_t)t * K + (int64_t)(kb0 + kbl) * 128 + (c & 7) * 16,
                          sX + row * Ld::XROWB + slot0 * 16);
            }
        }
        // activation scales [row][KMAX] (rows < nvp, K-blocks < nk), two per thread
        constexpr int XSPT = C::RP * C::KMAX / C::NT;
        float xs[XSPT], wsv = 0.f;
        int xsi[XSPT];
#pragma unroll
        for (int j = 0; j < XSPT; ++j) {
            const int idx = tid + j * C::NT;
            xs[j] = 0.f;
            xsi[j] = -1;
            if (idx < nvp * nk) {
                const int srow = idx / nk, skb = idx - srow * nk;
                if (sTok[srow] >= 0) {
                    xs[j] = a.xs[(int64_t)sXt[srow] * a.nkb + kb0 + skb];
                    xsi[j] = srow * C::KMAX + skb;
                }
            }
        }
        const int nb13 = (int)(2 * I / 128);
        const int half = tid / C::KMAX, wkb = tid % C::KMAX;   // half < 2: weight scale slot
        if (half < 2 && wkb < nk)
            wsv = a.w13s[((int64_t)e * nb13 + (half ? (int)(I / 128) : 0) + jt) * a.nkb + kb0 + wkb];
        // the weight stream starts behind the activation tile: waiting for
        // the tile then leaves both weight stages in flight
        issue(0, std::integral_constant<int, 0>{});
        issue(1, std::integral_constant<int, 1>{});
        wait_vmcnt<2 * C::LPS>();
#pragma unroll
        for (int j = 0; j < XSPT; ++j)
            if (xsi[j] >= 0) sXs[xsi[j]] = xs[j];
        if (half < 2) sWs[tid] = wsv;           // [half][KMAX]
    }
    __syncthreads();

    v4f accg[C::NU], accu[C::NU];
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        accg[u] = v4f{0.f, 0.f, 0.f, 0.f};
        accu[u] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // K-blocks past the range (the tail of the last stage, whole dummy
    // stages) carry zero scales, so they add exact zeros: their weights are
    // finite codes or zeros and the x tile holds finite codes up to the next
    // multiple of 8 K-blocks.
    auto compute = [&](int st, auto BUF) {
        constexpr int bf = decltype(BUF)::value;
#pragma unroll
        for (int kk = 0; kk < C::S; ++kk) {
            const int kbl = st * C::S + kk;
            const float sg = sWs[kbl], su = sWs[C::KMAX + kbl];
            v8h Wg[4], Wu[4];
            if constexpr (MODE == kExact) {
                e4m3x32_to_f16(wb[bf][kk][0], wb[bf][kk][1], Wg);
                e4m3x32_to_f16(wb[bf][kk][2], wb[bf][kk][3], Wu);
            }
#pragma unroll
            for (int u = 0; u < C::NU; ++u) {
                if (16 * u >= nvp) break;
                const int row = 16 * u + l16;
                const uint8_t *xp = sX + row * Ld::XROWB + kbl * 128;
                const u32x4 lo = lds_read16(xp + ((g ^ (row & 7)) << 4));
                const u32x4 hi = lds_read16(xp + (((4 + g) ^ (row & 7)) << 4));
                const float sa = sXs[row * C::KMAX + kbl];
                if constexpr (MODE == kExact) {
                    v8h Bh[4];
                    e4m3x32_to_f16(lo, hi, Bh);
                    const v4f tg = mfma16x16x128_f16(Wg, Bh);
                    const v4f tu = mfma16x16x128_f16(Wu, Bh);
                    accg[u] = tg * (sa * sg) + accg[u];
                    accu[u] = tu * (sa * su) + accu[u];
                } else {
                    const v8i B = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    const u32x4 &g0 = wb[bf][kk][0], &g1 = wb[bf][kk][1];
                    const u32x4 &u0 = wb[bf][kk][2], &u1 = wb[bf][kk][3];
                    const v8i Ag = {(int)g0.x, (int)g0.y, (int)g0.z, (int)g0.w,
                                    (int)g1.x, (int)g1.y, (int)g1.z, (int)g1.w};
                    const v8i Au = {(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                                    (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
                    if constexpr (MODE == kFp8E8) {
                        const int eb = e8m0_of(sa);
                        accg[u] = mfma16x16x128_e8m0(Ag, B, accg[u], e8m0_of(sg), eb);
                        accu[u] = mfma16x16x128_e8m0(Au, B, accu[u], e8m0_of(su), eb);
                    } else {
                        accg[u] = mfma16x16x128(Ag, B) * (sa * sg) + accg[u];
                        accu[u] = mfma16x16x128(Au, B) * (sa * su) + accu[u];
                    }
                }
            }
        }
    };
    // Stage st computes from buffer st & 1, then refills it with stage st + 2.
    // (pairs of stages, then an odd last one: no exit from the middle of
    // the loop body, which keeps the compiler's own waits at the stage
    // boundaries)
    int st = 0;
    for (; st + 1 < nst; st += 2) {
        wait_vmcnt<C::LPS>();
        compute(st, std::integral_constant<int, 0>{});
        issue(st + 2, std::integral_constant<int, 0>{});
        wait_vmcnt<C::LPS>();
        compute(st + 1, std::integral_constant<int, 1>{});
        issue(st + 3, std::integral_constant<int, 1>{});
    }
    if (st < nst) {
        wait_vmcnt<C::LPS>();
        compute(st, std::integral_constant<int, 0>{});
    }

    // ---- FP32 tile of the pass: sG[row][n], gate n < 128, up n >= 128
    __syncthreads();                            // every wave is done with the x tile
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        if (16 * u >= nvp) break;
        float *gp = sG + (16 * u + l16) * C::GROW + 16 * w + 4 * g;
        *reinterpret_cast<v4f *>(gp) = accg[u];
        *reinterpret_cast<v4f *>(gp + 128) = accu[u];
    }
    __syncthreads();

    if (a.nsplit > 1) {
        // Partial sums travel through memory with agent-coherent accesses
        // (sc1: stores write through this XCD's L2, loads miss in it), so the
        // hand-off needs only the stores' completion before the counter
        // bump -- no cache-wide write-back or invalidate.
        const int tile = jt * a.nblocks + b;
        const int sstride = BM * 256 * 4;       // bytes between splits
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.part + (size_t)tile * a.nsplit * BM * 256 + (size_t)row0 * 256), (short)0,
            a.nsplit * sstride, 0x00020000);
        constexpr int kAgent = 16;              // cache policy: sc1
        for (int idx = tid; idx < nvp * 64; idx += C::NT) {
            const int row = idx >> 6, c4 = idx & 63;
            if (sTok[row] >= 0)
                __builtin_amdgcn_raw_buffer_store_b128(
                    *reinterpret_cast<const u32x4 *>(sG + row * C::GROW + 4 * c4), rp,
                    split * sstride + (row * 256 + 4 * c4) * 4, 0, kAgent);
        }
        wait_vmcnt<0>();
        __syncthreads();
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(&a.cnt[tile * C::NPASS + pass], 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sMisc[1] = old == (unsigned)(a.nsplit - 1);
        }
        __syncthreads();
        if (!sMisc[1]) return;
        for (int idx = tid; idx < nvp * 64; idx += C::NT) {
            const int row = idx >> 6, c4 = idx & 63;
            if (sTok[row] < 0) continue;
            const int off = (row * 256 + 4 * c4) * 4;
            v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < a.nsplit; s0 += 16) {
                u32x4 v[16];
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (s0 + q < a.nsplit)
                        v[q] = __builtin_amdgcn_raw_buffer_load_b128(rp, (s0 + q) * sstride + off, 0, kAgent);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (s0 + q < a.nsplit) {
                        sum.x += __uint_as_float(v[q].x);
                        sum.y += __uint_as_float(v[q].y);
                        sum.z += __uint_as_float(v[q].z);
                        sum.w += __uint_as_float(v[q].w);
                    }
            }
            *reinterpret_cast<v4f *>(sG + row * C::GROW + 4 * c4) = sum;
        }
        __syncthreads();
    }

    // ---- SwiGLU + per-row 128-group FP8 requantisation: 32 lanes per row
    const bool ue = a.inter_ue8m0 != 0;
    for (int base = 0; base < nvpad * 32; base += C::NT) {
        const int idx = base + tid;
        const int row = idx >> 5, q = idx & 31;
        const float *gp = sG + row * C::GROW + 4 * q;
        const v4f gv = *reinterpret_cast<const v4f *>(gp);
        const v4f uv = *reinterpret_cast<const v4f *>(gp + 128);
        float h[4], amax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = swiglu(gv[i], uv[i]);
            amax = fmaxf(amax, fabsf(h[i]));
        }
        amax = wave_max_xor(amax, 1);
        amax = wave_max_xor(amax, 2);
        amax = wave_max_xor(amax, 4);
        amax = wave_max_xor(amax, 8);
        amax = wave_max_xor(amax, 16);
        float s, inv;
        group_scale(amax, ue, s, inv);
        if (row < nvp && sTok[row] >= 0) {
            const int64_t p = (int64_t)b * BM + row0 + row;
            *reinterpret_cast<uint32_t *>(a.hq + p * I + (int64_t)jt * 128 + 4 * q) =
                pack_e4m3x4(h[0] * inv, h[1] * inv, h[2] * inv, h[3] * inv);
            if (q == 0) a.hs[p * (I >> 7) + jt] = s;
        }
    }
}

template <int BM, int MODE>
hipError_t launch_gs(const GateUpArgs &a, hipStream_t st) {
    using C = GSCfg<BM>;
    const int64_t grid = (int64_t)a.nblocks * a.nsplit * a.jtiles * C::NPASS;
    if (grid == 0) return hipSuccess;
    if (a.kb_per_split < 1 || a.kb_per_split > C::KMAX) return hipErrorInvalidValue;
    const int lds = GSLayout<BM>::TOTAL;
    if (lds > 64 * 1024) {                      // once per device
        static bool attr_set[64] = {};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        if (!attr_set[dev]) {
            e = hipFuncSetAttribute((const void *)gateup_stream_kernel<BM, MODE>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            attr_set[dev] = true;
        }
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

}  // namespace

int gateup_stream_kmax(int block_m) { return 1024 / (block_m < 64 ? block_m : 64); }

hipError_t launch_gateup(const GateUpArgs &a, int block_m, bool fp8_mma, bool e8m0,
                         hipStream_t st) {
    const int mode = !fp8_mma ? kExact : (e8m0 ? kFp8E8 : kFp8);
    switch (block_m) {
        case 16: return launch_gs_mode<16>(a, mode, st);
        case 32: return launch_gs_mode<32>(a, mode, st);
        case 64: return launch_gs_mode<64>(a, mode, st);
        case 128: return launch_gs_mode<128>(a, mode, st);
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
