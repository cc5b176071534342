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

// bf16 workgroup tile: GATE_BM x 256 with waves of GATE_WM x 128 and
// GATE_WPE waves per SIMD.  Default: 256 x 256 with 8 waves of 64 x 128 (two
// per SIMD, so one wave's LDS reads and barrier waits overlap the other's
// MFMAs) fed by a 3-deep ring of 64-byte K stages (96 KiB of LDS).  A 256-wide
// tile moves 2/3 of the L2->LDS bytes per flop of a 128 x 256 one.
#ifndef GATE_BM
#define GATE_BM 256
#endif
#ifndef GATE_WPE
#define GATE_WPE 2
#endif
#ifndef GATE_WM
#define GATE_WM 64
#endif
#ifndef GATE_KB
#define GATE_KB 64
#endif
#ifndef GATE_STAGES
#define GATE_STAGES 3
#endif

namespace twell {

template <typename TI> struct TwellOut {
    TI *val;
    uint8_t *idx;
    int32_t *cnt;
    int cap, n_b;
};

// Pack the accumulators of one BM x BN output tile into TwELL (tile width TW).
// The unrolled part touches each accumulator register twice with a couple of
// instructions; everything that depends on the (few) active values runs in
// short loops, so the epilogue's code stays small next to the 64 KiB
// instruction cache a CU pair shares.
//   pass 1 (per wave): one ballot per accumulator register gives two rows'
//           32-bit activity masks for one 32-column block (the active test is
//           the fp32 accumulator > 0); the 16 registers' masks are gathered
//           into lanes 0-15 and stored as mask[row][block].
//   pass 2 (one thread per row): popcount of each tile's masks -> the true
//           count (stored, and kept in LDS).
//   pass 3, per 32-row block fm of every wave: the block's values, rounded to
//           the storage type, go to an LDS tile; then one thread per (row,
//           tile) walks the set mask bits in ascending column order and puts
//           the first `cap` (value, tile-local column) pairs in an LDS staging
//           row (or straight to memory when staging does not fit).
//   pass 4 (one thread per (row, tile)): staged slots go out with 16-byte
//           stores, slots past min(count, cap) as zeros.
template <typename TI, int BM, int BN, int WM, int WN, int TW, int LDS_BYTES>
__device__ __forceinline__ void twell_epilogue(f32x16 (&acc)[WM / 32][WN / 32], char *smem, int m0, int n0, int M,
                                               int N, const TwellOut<TI> &o)
{
    constexpr int FM = WM / 32, FN = WN / 32, NWN = BN / WN, NWM = BM / WM;
    constexpr int BPW = WN / 32;  // 32-column blocks per wave
    constexpr int BPT = TW / 32;  // 32-column blocks per TwELL tile
    constexpr int TPW = BN / TW;  // TwELL tiles per workgroup row
    constexpr int NTHR = NWM * NWN * 64;
    constexpr int SZ = sizeof(TI);
    constexpr int CROWS = NWM * 32;  // rows of one pass-3 block (block fm of every wave row)
    static_assert(BN / 32 == 8, "a row's masks are 8 words");
    static_assert(BN % TW == 0, "the workgroup's columns cover whole TwELL tiles");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;
    const int cap = o.cap;
    uint32_t *smask = reinterpret_cast<uint32_t *>(smem);        // [BM][8] block masks
    int16_t *scnt = reinterpret_cast<int16_t *>(smem + BM * 32);  // [BM][TPW] true counts
    constexpr int SV_OFF = BM * 32 + ((BM * TPW * 2 + 15) & ~15);
    TI *sv = reinterpret_cast<TI *>(smem + SV_OFF);               // [CROWS][BN] values of one block
    constexpr int STAGE_OFF = SV_OFF + CROWS * BN * SZ;
    char *stage = smem + STAGE_OFF;  // [BM][TPW][cap] values, then [BM][TPW][cap] indices
    const bool staged = STAGE_OFF + BM * TPW * cap * (SZ + 1) <= LDS_BYTES;
    static_assert(STAGE_OFF <= LDS_BYTES, "epilogue LDS");
    TI *sval = reinterpret_cast<TI *>(stage);
    uint8_t *sidx = reinterpret_cast<uint8_t *>(stage + BM * TPW * cap * SZ);

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
        const int t = m0 + r;
#pragma unroll
        for (int tl = 0; tl < TPW; ++tl) {
            int n = 0;
#pragma unroll
            for (int b = 0; b < BPT; ++b)
                n += __popc(smask[r * 8 + tl * BPT + b]);
            scnt[r * TPW + tl] = (int16_t)n;
            const int gcol = n0 + tl * TW;
            if (t < M && gcol < N)
                o.cnt[(int64_t)t * o.n_b + gcol / TW] = n;
        }
    }

    // pass 3
    const int lc = lane & 31;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        __syncthreads();  // sv is free (previous block consumed; pass 2 done)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * WN + fn * 32 + lc;
#pragma unroll
            for (int i = 0; i < 16; ++i)  // every value: only active positions are read back
                store_elem(sv + (wm * 32 + acc_row(i, lane)) * BN + col, acc[fm][fn][i]);
        }
        __syncthreads();
        for (int e = tid; e < CROWS * TPW; e += NTHR) {
            const int cr = e / TPW, tl = e - cr * TPW;  // row cr of the block: wave row cr / 32
            const int r = (cr >> 5) * WM + fm * 32 + (cr & 31);
            const int t = m0 + r;
            const int gbase = n0 + tl * TW;
            if (t >= M || gbase >= N)
                continue;
            const int off = (t * o.n_b + gbase / TW) * cap;
            const int so = (r * TPW + tl) * cap;
            int k = 0;
            for (int b = 0; b < BPT && k < cap; ++b) {
                uint32_t m = smask[r * 8 + tl * BPT + b];
                while (m != 0u && k < cap) {
                    const int c = b * 32 + __ffs(m) - 1;  // tile-local column, ascending
                    m &= m - 1u;
                    const TI v = sv[cr * BN + tl * TW + c];
                    if (staged) {
                        sval[so + k] = v;
                        sidx[so + k] = (uint8_t)c;
                    } else {
                        o.val[off + k] = v;
                        o.idx[off + k] = (uint8_t)c;
                    }
                    ++k;
                }
            }
        }
    }
    __syncthreads();

    // pass 4
    const bool vval = staged && (cap * SZ) % 16 == 0 && (reinterpret_cast<uintptr_t>(o.val) & 15u) == 0;
    const bool vidx = staged && cap % 8 == 0 && (reinterpret_cast<uintptr_t>(o.idx) & 7u) == 0;
    for (int e = tid; e < BM * TPW; e += NTHR) {
        const int r = e / TPW, tl = e - r * TPW;
        const int t = m0 + r;
        const int gcol = n0 + tl * TW;
        if (t >= M || gcol >= N)
            continue;
        const int kept = min((int)scnt[e], cap);
        const int off = (t * o.n_b + gcol / TW) * cap;
        if (vval) {
            const TI *svr = sval + e * cap;
            for (int s0 = 0; s0 < cap; s0 += 16 / SZ) {
                u32x4 w = *reinterpret_cast<const u32x4 *>(svr + s0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {  // zero the slots at or past `kept`
                    if constexpr (SZ == 2) {
                        const int sa = s0 + 2 * q;
                        w[q] &= (sa < kept ? 0xFFFFu : 0u) | (sa + 1 < kept ? 0xFFFF0000u : 0u);
                    } else {
                        w[q] = s0 + q < kept ? w[q] : 0u;
                    }
                }
                *reinterpret_cast<u32x4 *>(o.val + off + s0) = w;
            }
        } else {
            for (int s = 0; s < cap; ++s) {
                if (s < kept) {
                    if (staged)
                        o.val[off + s] = sval[e * cap + s];
                } else {
                    store_elem(o.val + off + s, 0.f);
                }
            }
        }
        if (vidx) {
            const uint8_t *si = sidx + e * cap;
            for (int s0 = 0; s0 < cap; s0 += 8) {
                uint2 w = *reinterpret_cast<const uint2 *>(si + s0);
                uint32_t k0 = 0, k1 = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    k0 |= (s0 + bb < kept ? 0xFFu : 0u) << (8 * bb);
                    k1 |= (s0 + 4 + bb < kept ? 0xFFu : 0u) << (8 * bb);
                }
                w.x &= k0;
                w.y &= k1;
                *reinterpret_cast<uint2 *>(o.idx + off + s0) = w;
            }
        } else {
            for (int s = 0; s < cap; ++s) {
                if (s < kept) {
                    if (staged)
                        o.idx[off + s] = sidx[e * cap + s];
                } else {
                    o.idx[off + s] = 0;
                }
            }
        }
    }
}

template <typename TI, int BM, int BN, int WM, int WN, int TW, int KB, int STAGES, int WPE>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
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
    twell_epilogue<TI, BM, BN, WM, WN, TW, Core::LDS_BYTES>(acc, smem, m0, n0, p.M, p.N, o);
}

template <typename TI, int BM, int BN, int WM, int WN, int KB, int STAGES, int WPE>
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
        gate_twell_kernel<TI, BM, BN, WM, WN, 32, KB, STAGES, WPE><<<grid, block, 0, s>>>(p, o);
        break;
    case 64:
        gate_twell_kernel<TI, BM, BN, WM, WN, 64, KB, STAGES, WPE><<<grid, block, 0, s>>>(p, o);
        break;
    case 128:
        gate_twell_kernel<TI, BM, BN, WM, WN, 128, KB, STAGES, WPE><<<grid, block, 0, s>>>(p, o);
        break;
    default:
        gate_twell_kernel<TI, BM, BN, WM, WN, 256, KB, STAGES, WPE><<<grid, block, 0, s>>>(p, o);
        break;
    }
    return hipGetLastError();
}

// Tile shapes: bf16 as configured above, fp32 64 x 256 (4 waves of 32 x 128).
hipError_t launch_gate_twell(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                             void *val, uint8_t *idx, int32_t *cnt, hipStream_t s)
{
    if (vdtype == 1)
        return gate_twell_go<__bf16, GATE_BM, 256, GATE_WM, 128, GATE_KB, GATE_STAGES, GATE_WPE>(x, wg_t, T, d, F,
                                                                                               tile_w, cap, val,
                                                                              idx, cnt, s);
    return gate_twell_go<float, 64, 256, 32, 128, 128, 2, 1>(x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, s);
}

}  // namespace twell
