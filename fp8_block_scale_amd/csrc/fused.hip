// Steps 3-5 in one launch: gate/up, SwiGLU + requantisation, down GEMM and
// the weighted route sum into the BF16 output, with no launch boundary
// between them (the single fused expert kernel of FlashInfer PR #4287, PR
// summary, whose SM100 design keeps the whole expert computation in one
// kernel; "Final W8 kernel performance (v46)" fuses all five of the stock
// kernels' stages into one).
//
// The MI355X design: one launch whose workgroups each run one work item,
// chosen by a ticket taken when the workgroup starts (not by its launch
// index).  Tickets come from 16 queues; queue q owns the plan blocks
// b = q (mod 16) and hands out their items in this order --
//   gate/up items of gateup_item.h (block, row pass, j-tile, K-split; split-K
//     partial sums go to the last arriver, which writes the intermediate rows
//     and bumps cnt_h);
//   down items of down_item.h (block, row pass, column group): the W2 stream
//     starts at once, the item then waits until its block's intermediate
//     rows are complete, multiplies, writes y and counts its rows per
//     (token, 256-column tile); the item that completes a (token, tile) adds
//     the token's route rows into the output in route order and rounds once.
// A down item waits only for gate/up items of its own block: lower tickets
// of its own queue, taken by workgroups that have started, are resident and
// never wait themselves, so every wait ends (and each wait is bounded
// besides, see wait_count).  The route map the route sum needs is built
// before the launch by a one-workgroup set-up kernel.  Two workgroups fit
// on a CU at decode sizes, so the W2 stream of the down items overlaps the
// W13 stream of the gate/up items.  Data handed between workgroups
// (split-K partials, intermediate rows, y) moves with agent-coherent
// accesses (common.h).
//
// Measured dead ends: a single ticket counter for the whole launch (every
// workgroup's first atomic serialises on one address: ~25-50 ns per
// workgroup, +17 us at decode M=1, +68 us at M=16), and a persistent
// variant looping over tickets (values of both item kinds stayed live
// across the loop: 165 VGPRs, one workgroup per CU).
//
// The arithmetic is the two-launch path's, item for item, so the output is
// bit-identical to it.
#include "down_item.h"
#include "gateup_item.h"

namespace moe {

namespace {

constexpr int kNT = 512;
#ifndef MOE_FUSED_GU_STAGES
#define MOE_FUSED_GU_STAGES 2
#endif
constexpr int kGuStages = MOE_FUSED_GU_STAGES;   // gate/up ring depth (two workgroups per CU)

// The set-up launch: one workgroup clears the counters and the route map,
// then writes the plan rows of the valid routes.
__global__ void __launch_bounds__(1024)
fused_prep_kernel(uint32_t *__restrict__ cnt, size_t n_cnt, int32_t *__restrict__ rpos, int64_t R,
                  const int32_t *__restrict__ sorted, const int32_t *__restrict__ ntp,
                  int64_t sorted_cap) {
    for (size_t i = threadIdx.x; i < n_cnt; i += 1024) cnt[i] = 0u;
    for (int64_t i = threadIdx.x; i < R; i += 1024) rpos[i] = -1;
    __syncthreads();
    const int64_t P = ntp[0] < sorted_cap ? ntp[0] : sorted_cap;
    for (int64_t p = threadIdx.x; p < P; p += 1024) {
        const int r = sorted[p];
        if (r >= 0 && (int64_t)r < R) rpos[r] = (int32_t)p;
    }
}

template <int BM, int GMODE, bool E8>
__global__ void __launch_bounds__(kNT)
fused_experts_kernel(GateUpArgs ga, DownArgs da, FusedArgs f) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int *sTicket = reinterpret_cast<int *>(smem + f.lds_ticket);   // past every item's LDS
    constexpr int NPASS = gs::GSCfg<BM, kGuStages>::NPASS;
    // workgroups go to the 8 XCDs round robin by launch index: eight
    // consecutive workgroups share a queue, so every queue's items (and
    // every block's) spread over all XCDs
    const int q = (blockIdx.x >> 3) % kFusedQueues;
    if (threadIdx.x == 0)
        *sTicket = (int)__hip_atomic_fetch_add(f.tickets + q, 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int t = *sTicket;
    const int nbq = (ga.nblocks - q + kFusedQueues - 1) / kFusedQueues;   // blocks of this queue
    const int n_gu = nbq * ga.nsplit * ga.jtiles * NPASS;
    if (t < n_gu) {
        const int bi = t % nbq;
        t /= nbq;
        const int split = t % ga.nsplit;
        t /= ga.nsplit;
        const int jt = t % ga.jtiles;
        const int pass = t / ga.jtiles;
        gs::gateup_item<BM, GMODE, kGuStages, true>(ga, smem, q + bi * kFusedQueues, split, jt,
                                                    pass, f.cnt_h);
        return;
    }
    t -= n_gu;
    const int ncw = (da.ctiles + da.nct - 1) / da.nct;
    if (t < nbq * ncw * NPASS) {
        const int bi = t % nbq;
        t /= nbq;
        const int cw = t % ncw;
        const int pass = t / ncw;
        ds::down_item<BM, E8, true>(da, smem, q + bi * kFusedQueues, cw, pass, &f);
    }
}

template <int BM>
int down_nct(const DownArgs &a) {
    using C = ds::DSCfg<BM>;
    const int64_t units = (int64_t)a.nblocks * a.ctiles * C::NPASS;
    int nct = (int)(units / 1024);
    return nct < 1 ? 1 : (nct > C::NCTMAX ? C::NCTMAX : nct);
}

template <int BM, int GMODE, bool E8>
hipError_t launch_fused_t(const GateUpArgs &ga, DownArgs da, FusedArgs f, hipStream_t st) {
    using G = gs::GSCfg<BM, kGuStages>;
    using D = ds::DSCfg<BM>;
    if (ga.nblocks == 0) return hipSuccess;
    if (da.njb > D::JMAX || ga.kb_per_split < 1) return hipErrorInvalidValue;
    da.nct = down_nct<BM>(da);
    const int64_t ncw = (da.ctiles + da.nct - 1) / da.nct;
    // the most blocks any queue owns (queue 0's)
    const int64_t nbq = (ga.nblocks + kFusedQueues - 1) / kFusedQueues;
    const int64_t per_q = nbq * ((int64_t)ga.nsplit * ga.jtiles * G::NPASS + ncw * D::NPASS);
    const int lds_d = ds::DSLayout(D::RP, da.njb, da.nct, D::YROW).total;
    f.lds_ticket = ((G::TOTAL > lds_d ? G::TOTAL : lds_d) + 15) & ~15;
    const int lds = f.lds_ticket + 16;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    // one item per workgroup; each run of 8 * kFusedQueues workgroups gives
    // every queue 8 of them
    const int64_t grid = (per_q + 7) / 8 * 8 * kFusedQueues;
    if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    f.per_queue = (int)per_q;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = raise_lds_limit(lds_set, (const void *)fused_experts_kernel<BM, GMODE, E8>, 160 * 1024);
    if (e != hipSuccess) return e;
    fused_experts_kernel<BM, GMODE, E8><<<(unsigned)grid, kNT, lds, st>>>(ga, da, f);
    return hipGetLastError();
}

template <int BM>
hipError_t launch_fused_bm(const GateUpArgs &ga, const DownArgs &da, const FusedArgs &f, bool fp8,
                           bool e8, hipStream_t st) {
    if (!fp8) return e8 ? launch_fused_t<BM, gs::kExactE8, true>(ga, da, f, st)
                        : launch_fused_t<BM, gs::kExact, false>(ga, da, f, st);
    return e8 ? launch_fused_t<BM, gs::kFp8E8, true>(ga, da, f, st)
              : launch_fused_t<BM, gs::kFp8, false>(ga, da, f, st);
}

}  // namespace

int fused_max_njb(int block_m) {
    switch (block_m) {
        case 8: return ds::DSCfg<8>::JMAX;
        case 16: return ds::DSCfg<16>::JMAX;
        case 32: return ds::DSCfg<32>::JMAX;
        case 64: return ds::DSCfg<64>::JMAX;
        case 128: return ds::DSCfg<128>::JMAX;
        default: return 0;
    }
}

size_t fused_counter_words(int64_t nblocks, int block_m, int64_t M, int64_t ctiles) {
    const int64_t npass = block_m > 64 ? block_m / 64 : 1;
    return kFusedQueues + 4 + (size_t)(nblocks * npass) + (size_t)(M * ctiles);
}

hipError_t launch_fused_prep(uint32_t *cnt, size_t n_cnt, int32_t *rpos, int64_t R,
                             const int32_t *sorted, const int32_t *ntp, int64_t sorted_cap,
                             hipStream_t st) {
    fused_prep_kernel<<<1, 1024, 0, st>>>(cnt, n_cnt, rpos, R, sorted, ntp, sorted_cap);
    return hipGetLastError();
}

hipError_t launch_fused(const GateUpArgs &ga, const DownArgs &da, const FusedArgs &f, int block_m,
                        bool fp8_mma, bool e8m0, hipStream_t st) {
    switch (block_m) {
        case 8: return launch_fused_bm<8>(ga, da, f, fp8_mma, e8m0, st);
        case 16: return launch_fused_bm<16>(ga, da, f, fp8_mma, e8m0, st);
        case 32: return launch_fused_bm<32>(ga, da, f, fp8_mma, e8m0, st);
        case 64: return launch_fused_bm<64>(ga, da, f, fp8_mma, e8m0, st);
        case 128: return launch_fused_bm<128>(ga, da, f, fp8_mma, e8m0, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
