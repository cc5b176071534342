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

namespace twell {

template <typename TI> struct TwellOut {
    TI *val;
    uint8_t *idx;
    int32_t *cnt;
    int tile_w, cap, n_b;
};

// Pack the accumulators of one BM x BN output tile into TwELL.
template <typename TI, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void twell_epilogue(f32x16 (&acc)[WM / 32][WN / 32], char *smem, int m0, int n0, int M,
                                               int N, const TwellOut<TI> &o)
{
    constexpr int FM = WM / 32, FN = WN / 32, NWN = BN / WN;
    constexpr int NBLK = BN / 32;
    static_assert(NBLK <= 8, "row block counts are read as one 8-byte word");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / NWN, wn = wave % NWN;
    uint8_t *pc = reinterpret_cast<uint8_t *>(smem);  // [BM][8] active count per 32-column block

    // Pass 1: per (row, 32-column block) active counts.
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int blk = (wn * WN + fn * 32) >> 5;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint64_t mask = __ballot(acc[fm][fn][i] > 0.f);
                if (lane == 0) {
                    const int r = wm * WM + fm * 32 + acc_row(i, 0);
                    pc[r * 8 + blk] = (uint8_t)__popc((uint32_t)mask);
                    pc[(r + 4) * 8 + blk] = (uint8_t)__popc((uint32_t)(mask >> 32));
                }
            }
        }
    __syncthreads();

    // Pass 2: slots, values, indices and true counts.
    const int bpt = o.tile_w >> 5;  // 32-column blocks per TwELL tile
    const int lh = lane >> 5, lc = lane & 31;
    const uint32_t below = (1u << lc) - 1u;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int blk = (wn * WN + fn * 32) >> 5;
            const int tfirst = blk - blk % bpt;
            const int gcol = n0 + blk * 32 + lc;
            const int btile = gcol / o.tile_w;
            const int cloc = gcol - btile * o.tile_w;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float v = acc[fm][fn][i];
                const bool act = v > 0.f;
                const uint64_t mask = __ballot(act);
                const int r = wm * WM + fm * 32 + acc_row(i, lane);
                const uint64_t rowc = *reinterpret_cast<const uint64_t *>(pc + r * 8);
                int prefix = 0, total = 0;
#pragma unroll
                for (int b = 0; b < NBLK; ++b) {
                    const int cb = (int)((rowc >> (8 * b)) & 0xFF);
                    if (b >= tfirst && b < blk)
                        prefix += cb;
                    if (b >= tfirst && b < tfirst + bpt)
                        total += cb;
                }
                const uint32_t rm = lh ? (uint32_t)(mask >> 32) : (uint32_t)mask;
                const int slot = prefix + __popc(rm & below);
                const int t = m0 + r;
                if (t < M && gcol < N) {
                    const int64_t base = ((int64_t)t * o.n_b + btile) * o.cap;
                    if (act && slot < o.cap) {
                        store_elem(o.val + base + slot, v);
                        o.idx[base + slot] = (uint8_t)cloc;
                    }
                    if (lc == 0 && blk == tfirst)
                        o.cnt[(int64_t)t * o.n_b + btile] = total;
                }
            }
        }
}

template <typename TI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void gate_twell_kernel(GemmArgs p, TwellOut<TI> o)
{
    using Core = GemmCore<TI, BM, BN, WM, WN, false>;
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    int mt, nt;
    tile_coords(blockIdx.x, p.MT, p.NT, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    Core core;
    f32x16 acc[Core::FM][Core::FN];
    core.run(p, smem, m0, n0, p.M, p.k_begin, p.k_len, threadIdx.x, acc);
    twell_epilogue<TI, BM, BN, WM, WN>(acc, smem, m0, n0, p.M, p.N, o);
}

template <typename TI, int BM, int BN, int WM, int WN>
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
    TwellOut<TI> o{static_cast<TI *>(val), idx, cnt, tile_w, cap, F / tile_w};
    constexpr int NTHR = (BM / WM) * (BN / WN) * 64;
    gate_twell_kernel<TI, BM, BN, WM, WN><<<dim3(p.MT * p.NT), dim3(NTHR), 0, s>>>(p, o);
    return hipGetLastError();
}

hipError_t launch_gate_twell(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                             void *val, uint8_t *idx, int32_t *cnt, hipStream_t s)
{
    if (vdtype == 1)
        return gate_twell_go<__bf16, 256, 256, 128, 128>(x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, s);
    return gate_twell_go<float, 64, 256, 32, 128>(x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, s);
}

}  // namespace twell
