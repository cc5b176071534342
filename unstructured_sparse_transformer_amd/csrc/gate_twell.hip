// gate_twell.hip -- gate GEMM z = x . W_g with the TwELL epilogue.
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), section 2.1: TwELL cuts the hidden columns into tiles and packs
// each row's nonzeros per tile with tile-local indices; because the packing is
// tile-local, the gate matmul can emit it straight from its epilogue, after
// ReLU, with no extra launch, synchronisation or pass over memory.
//
// On gfx950 the workgroup's N extent (256 columns) always covers whole TwELL
// tiles, so the packing needs no cross-workgroup merge and is deterministic.
// The epilogue works straight on the MFMA accumulators: one ballot per
// accumulator register gives two rows' 32-column activity masks; their
// popcounts go through LDS to form, per row and tile, the prefix over the
// tile's 32-column blocks; each active lane then gets its slot as prefix +
// popcount of the lower lanes of its row mask (ascending column order).
#include "launch.h"
#include "twell_device.h"

#ifndef GATE_KB
#define GATE_KB 128
#endif
#ifndef GATE_STAGES
#define GATE_STAGES 2
#endif

namespace twell {

template <typename TI> struct TwellOut {
    TI *val;
    uint8_t *idx;
    int32_t *cnt;
    int cap, n_b;
};

// Pack the accumulators of one BM x BN output tile into TwELL (tile width TW).
//   pass 1 (per wave): one ballot per accumulator register gives two rows'
//           32-bit activity masks for one 32-column block; the 16 registers'
//           masks are gathered into lanes 0-15 and stored as mask[row][block].
//   pass 2 (one thread per row): popcounts of the row's 8 block masks ->
//           the exclusive prefix of each block inside its TwELL tile (kept in
//           LDS as bytes) and the true count of each tile (stored to memory).
//   pass 3 (per wave): registers whose ballot is empty -- most of them, the
//           activations being >99% zero -- are skipped with one wave-uniform
//           test; in the others every active lane stores its value and
//           tile-local index at slot = prefix + popcount(lower lanes of its
//           row's mask), i.e. in ascending column order.
template <typename TI, int BM, int BN, int WM, int WN, int TW>
__device__ __forceinline__ void twell_epilogue(f32x16 (&acc)[WM / 32][WN / 32], char *smem, int m0, int n0, int M,
                                               int N, const TwellOut<TI> &o)
{
    constexpr int FM = WM / 32, FN = WN / 32, NWN = BN / WN;
    constexpr int BPW = WN / 32;  // 32-column blocks per wave
    constexpr int BPT = TW / 32;  // 32-column blocks per TwELL tile
    constexpr int NTHR = (BM / WM) * NWN * 64;
    static_assert(BN / 32 == 8, "a row's masks are read as 8 words");
    static_assert(BN % TW == 0, "the workgroup's columns cover whole TwELL tiles");
    static_assert(BM % NTHR == 0 || NTHR % BM == 0, "rows per thread");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / NWN, wn = wave % NWN;
    uint32_t *smask = reinterpret_cast<uint32_t *>(smem);       // [BM][8] block masks
    uint8_t *spre = reinterpret_cast<uint8_t *>(smem + BM * 32);  // [BM][8] in-tile prefixes

    // pass 1
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            int vlo = 0, vhi = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint64_t mask = __ballot(acc[fm][fn][i] > 0.f);
                vlo = lane == i ? (int)(uint32_t)mask : vlo;
                vhi = lane == i ? (int)(uint32_t)(mask >> 32) : vhi;
            }
            if (lane < 16) {
                const int r = wm * WM + fm * 32 + acc_row(lane, 0);
                const int blk = wn * BPW + fn;
                smask[r * 8 + blk] = (uint32_t)vlo;
                smask[(r + 4) * 8 + blk] = (uint32_t)vhi;
            }
        }
    __syncthreads();

    // pass 2
    for (int r = tid; r < BM; r += NTHR) {
        const u32x4 mlo = *reinterpret_cast<const u32x4 *>(smask + r * 8);
        const u32x4 mhi = *reinterpret_cast<const u32x4 *>(smask + r * 8 + 4);
        const uint32_t mk[8] = {mlo[0], mlo[1], mlo[2], mlo[3], mhi[0], mhi[1], mhi[2], mhi[3]};
        uint32_t pw[2] = {0u, 0u};
        int run = 0;
        const int t = m0 + r;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            if (b % BPT == 0)
                run = 0;
            pw[b >> 2] |= (uint32_t)run << (8 * (b & 3));
            run += __popc(mk[b]);
            if (b % BPT == BPT - 1) {
                const int gcol = n0 + (b - BPT + 1) * 32;
                if (t < M && gcol < N)
                    o.cnt[(int64_t)t * o.n_b + gcol / TW] = run;
            }
        }
        *reinterpret_cast<uint2 *>(spre + r * 8) = make_uint2(pw[0], pw[1]);
    }
    __syncthreads();

    // pass 3
    const int lc = lane & 31, lh = lane >> 5;
    const uint64_t below = (1ull << lc) - 1ull;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int blk = wn * BPW + fn;
            const int gcol = n0 + blk * 32 + lc;
            const int btile = (n0 + blk * 32) / TW;
            const int cloc = gcol - btile * TW;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float v = acc[fm][fn][i];
                const bool act = v > 0.f;
                const uint64_t mask = __ballot(act);
                if (mask != 0ull) {
                    const int r = wm * WM + fm * 32 + acc_row(i, lane);
                    const int t = m0 + r;
                    const uint32_t rm = (uint32_t)(lh ? (mask >> 32) : mask);
                    const int slot = spre[r * 8 + blk] + __popc(rm & (uint32_t)below);
                    if (act && slot < o.cap && t < M && gcol < N) {
                        const int64_t off = ((int64_t)t * o.n_b + btile) * o.cap + slot;
                        store_elem(o.val + off, v);
                        o.idx[off] = (uint8_t)cloc;
                    }
                }
            }
        }
}

template <typename TI, int BM, int BN, int WM, int WN, int TW, int KB, int STAGES>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gate_twell_kernel(GemmArgs p, TwellOut<TI> o)
{
    using Core = GemmCore<TI, BM, BN, WM, WN, false, KB, STAGES>;
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    int mt, nt;
    tile_coords(blockIdx.x, p.MT, p.NT, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    Core core;
    f32x16 acc[Core::FM][Core::FN];
    core.run(p, smem, m0, n0, p.M, p.k_begin, p.k_len, threadIdx.x, acc);
    twell_epilogue<TI, BM, BN, WM, WN, TW>(acc, smem, m0, n0, p.M, p.N, o);
}

template <typename TI, int BM, int BN, int WM, int WN, int KB, int STAGES>
static hipError_t gate_twell_go(const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap, void *val,
                                uint8_t *idx, int32_t *cnt, hipStream_t s)
{
    GemmArgs p{};
    p.A = x;
    p.lda = d;
    p.M = T;
    p.B = wg_t;
    p.ldb = d;
    p.N = F;
    p.k_begin = 0;
    p.k_len = d;
    p.MT = (T + BM - 1) / BM;
    p.NT = (F + BN - 1) / BN;
    p.a_bytes = (uint32_t)((int64_t)T * d * sizeof(TI));
    p.b_bytes = (uint32_t)((int64_t)F * d * sizeof(TI));
    TwellOut<TI> o{static_cast<TI *>(val), idx, cnt, cap, F / tile_w};
    constexpr int NTHR = (BM / WM) * (BN / WN) * 64;
    const dim3 grid(p.MT * p.NT), block(NTHR);
    switch (tile_w) {
    case 32:
        gate_twell_kernel<TI, BM, BN, WM, WN, 32, KB, STAGES><<<grid, block, 0, s>>>(p, o);
        break;
    case 64:
        gate_twell_kernel<TI, BM, BN, WM, WN, 64, KB, STAGES><<<grid, block, 0, s>>>(p, o);
        break;
    case 128:
        gate_twell_kernel<TI, BM, BN, WM, WN, 128, KB, STAGES><<<grid, block, 0, s>>>(p, o);
        break;
    default:
        gate_twell_kernel<TI, BM, BN, WM, WN, 256, KB, STAGES><<<grid, block, 0, s>>>(p, o);
        break;
    }
    return hipGetLastError();
}

// Tile shapes: bf16 256 x 256 per workgroup (4 waves of 128 x 128, 256
// accumulator registers each), fp32 64 x 256.
hipError_t launch_gate_twell(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                             void *val, uint8_t *idx, int32_t *cnt, hipStream_t s)
{
    if (vdtype == 1)
        return gate_twell_go<__bf16, 256, 256, 128, 128, GATE_KB, GATE_STAGES>(x, wg_t, T, d, F, tile_w, cap, val,
                                                                              idx, cnt, s);
    return gate_twell_go<float, 64, 256, 32, 128, 128, 2>(x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, s);
}

}  // namespace twell
