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
// accumulator register gives two rows' activity over 32 columns, and each
// active lane's slot is the count of active columns before it in its tile
// (ascending column order).  Two forms: a single pass that fills per-wave
// segments of each row's tile in LDS (the common case), and a four-pass form
// (masks, per-row prefixes, placement, write-out) for capacities whose
// staging would not fit in LDS.
#include "launch.h"
#include "twell_device.h"

// bf16 workgroup tile: GATE_BM x 256 with waves of GATE_WM x 128 and
// GATE_WPE waves per SIMD.  Default: 256 x 256 with 8 waves of 64 x 128 (two
// per SIMD, so one wave's LDS reads and barrier waits overlap the other's
// MFMAs) fed by a 2-deep ring of 128-byte K stages (128 KiB of LDS), the
// copies of each stage spread between the MFMAs of the two sub-steps around
// the stage barrier (a burst of all 64 of a CU's 1 KiB copies right after the
// barrier kept waves from their MFMAs; spread: 3-4% faster).  A 256-wide tile
// moves 2/3 of the L2->LDS bytes per flop of a 128 x 256 one.
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

// One staged TwELL slot: the stored value's bits with the tile-local column
// above them (bf16: one 32-bit word; fp32: one 64-bit word).
template <typename TI> struct StageWord;
template <> struct StageWord<__bf16> {
    using W = uint32_t;
    __device__ static W pack(float v, int c)
    {
        const __bf16 h = (__bf16)v;
        return (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)c << 16);
    }
    // hi16: the column already shifted to bits 16..23
    __device__ static W pack_hi(float v, uint32_t hi16)
    {
        const __bf16 h = (__bf16)v;
        return (uint32_t)__builtin_bit_cast(uint16_t, h) | hi16;
    }
    __device__ static uint32_t bits(W w) { return w & 0xFFFFu; }
    __device__ static uint32_t col(W w) { return w >> 16; }
};
template <> struct StageWord<float> {
    using W = uint64_t;
    __device__ static W pack(float v, int c) { return (uint64_t)__float_as_uint(v) | ((uint64_t)c << 32); }
    __device__ static W pack_hi(float v, uint32_t hi16)
    {
        return (uint64_t)__float_as_uint(v) | ((uint64_t)(hi16 >> 16) << 32);
    }
    __device__ static uint32_t bits(W w) { return (uint32_t)w; }
    __device__ static uint32_t col(W w) { return (uint32_t)(w >> 32); }
};

// Pack the accumulators of one BM x BN output tile into TwELL (tile width TW).
// Every active value goes to its slot straight from the MFMA accumulators,
// in parallel: the slot of the value at (row, column c) is the number of
// active columns of the row that precede c inside c's TwELL tile.
//   pass 1 (per wave): one ballot per accumulator register gives two rows'
//           32-bit activity masks for one 32-column block (the active test is
//           the fp32 accumulator > 0); the 16 registers' masks are gathered
//           into lanes 0-15 and stored as mask[row][block].
//   pass 2 (one thread per row): per tile, the popcount of its blocks' masks
//           is the true count (stored, and kept in LDS); per block, the
//           exclusive prefix of the popcounts inside its tile (a byte).
//   pass 3 (per wave, per accumulator register): from its row's block mask
//           each lane gets its rank among the active columns below it; slot =
//           block prefix + rank.  Active values with slot < cap are written,
//           rounded to the storage type and packed with their tile-local
//           column, to an LDS staging row (or straight to memory when staging
//           does not fit).
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
    using SW = StageWord<TI>;
    using W = typename SW::W;
    static_assert(BN / 32 == 8, "a row's masks are 8 words");
    static_assert(BPW == 4, "a wave's blocks are one mask vector and one prefix word");
    static_assert(BN % TW == 0, "the workgroup's columns cover whole TwELL tiles");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;
    const int cap = o.cap;
    uint32_t *smask = reinterpret_cast<uint32_t *>(smem);            // [BM][8] block masks
    uint32_t *spre = reinterpret_cast<uint32_t *>(smem + BM * 32);   // [BM][2] prefix bytes
    int16_t *scnt = reinterpret_cast<int16_t *>(smem + BM * 40);     // [BM][TPW] true counts
    constexpr int STAGE_OFF = BM * 40 + ((BM * TPW * 2 + 15) & ~15);
    W *sw = reinterpret_cast<W *>(smem + STAGE_OFF);                 // [BM][TPW][cap] staged slots
    const bool staged = STAGE_OFF + BM * TPW * cap * (int)sizeof(W) <= LDS_BYTES;
    static_assert(STAGE_OFF <= LDS_BYTES, "epilogue LDS");

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
        uint32_t pre[2] = {0u, 0u};
        int run = 0;
        const int t = m0 + r;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            if (b % BPT == 0)
                run = 0;
            pre[b >> 2] |= (uint32_t)run << (8 * (b & 3));
            run += __popc(b < 4 ? mlo[b] : mhi[b - 4]);
            if (b % BPT == BPT - 1) {
                const int tl = b / BPT;
                scnt[r * TPW + tl] = (int16_t)run;
                const int gcol = n0 + tl * TW;
                if (t < M && gcol < N)
                    o.cnt[(int64_t)t * o.n_b + gcol / TW] = run;
            }
        }
        spre[r * 2] = pre[0];
        spre[r * 2 + 1] = pre[1];
    }
    __syncthreads();

    // pass 3
    const int lc = lane & 31;
    const uint32_t below = (1u << lc) - 1u;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = wm * WM + fm * 32 + acc_row(i, lane);
            // this half-wave's row: the wave's four block masks and their prefixes
            const u32x4 mw = *reinterpret_cast<const u32x4 *>(smask + r * 8 + wn * 4);
            const uint32_t pw = spre[r * 2 + wn];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint32_t m = mw[fn];
                const int slot = (int)((pw >> (8 * fn)) & 0xFFu) + __popc(m & below);
                if (((m >> lc) & 1u) && slot < cap) {
                    const float v = acc[fm][fn][i];
                    const int blk = wn * BPW + fn, tl = blk / BPT;
                    const int c = (blk % BPT) * 32 + lc;
                    if (staged) {
                        sw[(r * TPW + tl) * cap + slot] = SW::pack(v, c);
                    } else {
                        const int t = m0 + r, gcol = n0 + tl * TW;
                        if (t < M && gcol < N) {
                            const int64_t off = ((int64_t)t * o.n_b + gcol / TW) * cap + slot;
                            store_elem(o.val + off, v);
                            o.idx[off] = (uint8_t)c;
                        }
                    }
                }
            }
        }
    __syncthreads();

    // pass 4
    const bool vec = staged && (cap * SZ) % 16 == 0 && cap % 16 == 0 &&
                     (reinterpret_cast<uintptr_t>(o.val) & 15u) == 0 && (reinterpret_cast<uintptr_t>(o.idx) & 15u) == 0;
    for (int e = tid; e < BM * TPW; e += NTHR) {
        const int r = e / TPW, tl = e - r * TPW;
        const int t = m0 + r;
        const int gcol = n0 + tl * TW;
        if (t >= M || gcol >= N)
            continue;
        const int kept = min((int)scnt[e], cap);
        const int64_t off = ((int64_t)t * o.n_b + gcol / TW) * cap;
        const W *sr = sw + e * cap;
        if (vec) {
            // 16 slots at a time: 16 indices (one 16-byte store) and 16 values
            for (int s0 = 0; s0 < cap; s0 += 16) {
                u32x4 iw = {0u, 0u, 0u, 0u};
                uint32_t vb[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const bool k = s0 + q < kept;
                    const W w = k ? sr[s0 + q] : (W)0;
                    vb[q] = SW::bits(w);
                    iw[q >> 2] |= (k ? SW::col(w) : 0u) << (8 * (q & 3));
                }
                *reinterpret_cast<u32x4 *>(o.idx + off + s0) = iw;
                if constexpr (SZ == 2) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        u32x4 v;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[q] = vb[h * 8 + 2 * q] | (vb[h * 8 + 2 * q + 1] << 16);
                        *reinterpret_cast<u32x4 *>(o.val + off + s0 + h * 8) = v;
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        u32x4 v;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[q] = vb[h * 4 + q];
                        *reinterpret_cast<u32x4 *>(o.val + off + s0 + h * 4) = v;
                    }
                }
            }
        } else {
            for (int s = 0; s < cap; ++s) {
                if (s < kept) {
                    if (staged) {
                        const W w = sr[s];
                        if constexpr (SZ == 2)
                            reinterpret_cast<uint16_t *>(o.val)[off + s] = (uint16_t)SW::bits(w);
                        else
                            reinterpret_cast<uint32_t *>(o.val)[off + s] = SW::bits(w);
                        o.idx[off + s] = (uint8_t)SW::col(w);
                    }
                } else {
                    store_elem(o.val + off + s, 0.f);
                    o.idx[off + s] = 0;
                }
            }
        }
    }
}

// Segment form of the epilogue, used when the staging below fits in LDS.
// A segment is the part of one row's TwELL tile that one wave holds (the whole
// tile when the tile is no wider than a wave's columns, else a wave's share);
// a single pass over the accumulators fills every segment, so the ballots are
// taken once and only the (few) active values cost more than a compare.
//   pass A (per wave, per accumulator register): the ballot gives two rows'
//           32-bit activity masks for one 32-column block; a running count
//           over the wave's blocks gives each active lane its rank inside its
//           segment; active values with rank < cap are packed with their
//           tile-local column into the segment's staging slots; the
//           segments' true counts go to LDS.  All-zero ballots (most of them)
//           skip the rest.
//   pass B (one thread per 8 slots of a (row, tile)): the tile's segments
//           are joined in column order (the true count is their sum), and the
//           first `cap` slots go out with 16-byte value and 8-byte index
//           stores, slots past min(count, cap) as zeros.
template <typename TI, int BN, int WN, int TW> struct SegShape {
    static constexpr int SEGW = TW < WN ? TW : WN;  // columns of a segment
    static constexpr int NSEG = BN / SEGW;          // segments per row
    static constexpr int SPT = TW / SEGW;           // segments per tile
    static constexpr int BPS = SEGW / 32;           // 32-column blocks per segment
};
template <typename TI, int BM, int BN, int WN, int TW, int LDS_BYTES>
__host__ __device__ constexpr int seg_stage_off()
{
    return (BM * SegShape<TI, BN, WN, TW>::NSEG * 2 + 15) & ~15;
}
template <typename TI, int BM, int BN, int WN, int TW, int LDS_BYTES>
__device__ __forceinline__ bool seg_fits(int cap)
{
    return seg_stage_off<TI, BM, BN, WN, TW, LDS_BYTES>() +
               BM * SegShape<TI, BN, WN, TW>::NSEG * cap * (int)sizeof(typename StageWord<TI>::W) <=
           LDS_BYTES;
}

template <typename TI, int BM, int BN, int WM, int WN, int TW, int LDS_BYTES>
__device__ __forceinline__ void twell_epilogue_seg(f32x16 (&acc)[WM / 32][WN / 32], char *smem, int m0, int n0, int M,
                                                   int N, const TwellOut<TI> &o)
{
    constexpr int FM = WM / 32, FN = WN / 32, NWN = BN / WN, NWM = BM / WM;
    constexpr int NTHR = NWM * NWN * 64;
    constexpr int SZ = sizeof(TI);
    constexpr int TPW = BN / TW;
    using SS = SegShape<TI, BN, WN, TW>;
    constexpr int NSEG = SS::NSEG, SPT = SS::SPT, BPS = SS::BPS, SEGW = SS::SEGW;
    static_assert(SPT <= 2, "a tile spans at most two waves");
    using SW = StageWord<TI>;
    using W = typename SW::W;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;
    const int cap = o.cap;
    int16_t *scnt = reinterpret_cast<int16_t *>(smem);  // [BM][NSEG] segment true counts
    W *sw = reinterpret_cast<W *>(smem + seg_stage_off<TI, BM, BN, WN, TW, LDS_BYTES>());  // [BM][NSEG][cap]

    // pass A
    const int lc = lane & 31;
    const uint32_t lc16 = (uint32_t)lc << 16;
    const bool lo_half = lane < 32;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        int cnt_lo[FN / BPS], cnt_hi[FN / BPS];  // lanes i (0..15) collect register i's row counts
#pragma unroll
        for (int q = 0; q < FN / BPS; ++q)
            cnt_lo[q] = cnt_hi[q] = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = wm * WM + fm * 32 + acc_row(i, lane);
            uint32_t pre_lo = 0, pre_hi = 0;
            // all FN ballots first, so that each scalar test below reads a mask
            // whose compare has long finished
            uint64_t bal[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bal[fn] = __ballot(acc[fm][fn][i] > 0.f);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if (fn % BPS == 0)
                    pre_lo = pre_hi = 0;
                const float v = acc[fm][fn][i];
                const bool act = v > 0.f;
                const uint64_t b = bal[fn];
                const uint32_t blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
                if (b != 0u) {
                    // pre + active lanes of this row below the lane: mbcnt counts the
                    // set bits below the lane over all 64 lanes, so the upper half
                    // starts from pre_hi minus the lower half's count.
                    const int base = lo_half ? (int)pre_lo : (int)pre_hi - __popc(blo);
                    const int slot = __builtin_amdgcn_mbcnt_hi(bhi, __builtin_amdgcn_mbcnt_lo(blo, base));
                    if (act && slot < cap) {
                        const int col = wn * WN + fn * 32;  // first column of the block in the workgroup
                        const int seg = col / SEGW;
                        sw[(r * NSEG + seg) * cap + slot] = SW::pack_hi(v, ((uint32_t)(col % TW) << 16) | lc16);
                    }
                    pre_lo += __popc(blo);
                    pre_hi += __popc(bhi);
                }
                if (fn % BPS == BPS - 1) {
                    cnt_lo[fn / BPS] = lane == i ? (int)pre_lo : cnt_lo[fn / BPS];
                    cnt_hi[fn / BPS] = lane == i ? (int)pre_hi : cnt_hi[fn / BPS];
                }
            }
        }
        if (lane < 16) {
            const int r = wm * WM + fm * 32 + acc_row(lane, 0);
#pragma unroll
            for (int q = 0; q < FN / BPS; ++q) {
                const int seg = (wn * WN) / SEGW + q;
                scnt[r * NSEG + seg] = (int16_t)cnt_lo[q];
                scnt[(r + 4) * NSEG + seg] = (int16_t)cnt_hi[q];
            }
        }
    }
    __syncthreads();

    // pass B: 8-slot units, so that every thread has a unit (two per (row,
    // tile) at cap 16) and each unit goes out as one 16-byte (bf16) or two
    // (fp32) value stores and one 8-byte index store; other capacities and
    // unaligned buffers take one slot at a time.
    const bool vec8 = cap % 8 == 0 && (reinterpret_cast<uintptr_t>(o.val) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(o.idx) & 7u) == 0;
    const int U = vec8 ? cap >> 3 : 1;  // units per (row, tile)
    for (int e = tid; e < BM * TPW * U; e += NTHR) {
        const int rt = e / U, u = e - rt * U;
        const int r = rt / TPW, tl = rt - r * TPW;
        const int t = m0 + r;
        const int gcol = n0 + tl * TW;
        if (t >= M || gcol >= N)
            continue;
        const int s0 = r * NSEG + tl * SPT;  // first segment of the tile
        const int c0 = scnt[s0];
        const int c1 = SPT == 2 ? (int)scnt[s0 + 1] : 0;
        const int total = c0 + c1;
        const int64_t ooff = (int64_t)t * o.n_b + gcol / TW;
        if (u == 0)
            o.cnt[ooff] = total;
        const int k0 = min(c0, cap);  // slots taken from the first segment
        const int kept = min(total, cap);
        const W *sr0 = sw + (int64_t)s0 * cap;
        const W *sr1 = sr0 + cap;     // second segment (SPT == 2)
        const int64_t off = ooff * cap;
        if (vec8) {
            const int b0 = u * 8;
            uint32_t vb[8], iw[2] = {0u, 0u};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int sl = b0 + q;
                W w = (W)0;
                if (sl < k0)
                    w = sr0[sl];
                else if (SPT == 2 && sl < kept)
                    w = sr1[sl - k0];
                vb[q] = SW::bits(w);
                iw[q >> 2] |= (sl < kept ? SW::col(w) : 0u) << (8 * (q & 3));
            }
            *reinterpret_cast<uint2 *>(o.idx + off + b0) = make_uint2(iw[0], iw[1]);
            if constexpr (SZ == 2) {
                *reinterpret_cast<u32x4 *>(o.val + off + b0) =
                    u32x4{vb[0] | (vb[1] << 16), vb[2] | (vb[3] << 16), vb[4] | (vb[5] << 16), vb[6] | (vb[7] << 16)};
            } else {
                *reinterpret_cast<u32x4 *>(o.val + off + b0) = u32x4{vb[0], vb[1], vb[2], vb[3]};
                *reinterpret_cast<u32x4 *>(o.val + off + b0 + 4) = u32x4{vb[4], vb[5], vb[6], vb[7]};
            }
        } else {
            for (int sl = 0; sl < cap; ++sl) {
                W w = (W)0;
                if (sl < k0)
                    w = sr0[sl];
                else if (SPT == 2 && sl < kept)
                    w = sr1[sl - k0];
                if constexpr (SZ == 2)
                    reinterpret_cast<uint16_t *>(o.val)[off + sl] = (uint16_t)SW::bits(w);
                else
                    reinterpret_cast<uint32_t *>(o.val)[off + sl] = SW::bits(w);
                o.idx[off + sl] = (uint8_t)(sl < kept ? SW::col(w) : 0u);
            }
        }
    }
}

// Activation statistics of the gate (section 2.4 of the page: the L1
// penalty on the activations that training adds, and the neurons it leaves
// dead), gathered from the same accumulators before the packing.
struct GateStats {
    int32_t *neuron_cnt;  // [N]: rows with z > 0 per neuron, added atomically
    float *l1;            // [M][n_b]: sum of the positive z of each (row, tile)
};

// v from the lane whose index differs in bit log2(MASK) (inside 32 lanes):
// DPP for 1, 2 (quad permutes) and 8 (row rotate by 8), ds_swizzle's xor
// mode for 4 and 16.
template <int MASK> __device__ __forceinline__ float lane_xor(float v)
{
    const int b = __float_as_int(v);
    int r;
    if constexpr (MASK == 1)
        r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false);
    else if constexpr (MASK == 2)
        r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false);
    else if constexpr (MASK == 8)
        r = __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false);
    else
        r = __builtin_amdgcn_ds_swizzle(b, 0x1F | (MASK << 10));
    return __int_as_float(r);
}

// One halving step of a transposing reduction: lanes with bit BIT clear keep
// registers [0, N) and lanes with it set keep [N, 2N); each adds its partner's
// copy of the registers it keeps.
// (The lane test is a constant lane mask in SGPRs, not a per-lane value:
// per-lane lane bits would be long-lived VGPRs.)
template <int BIT> __device__ __forceinline__ float lane_bit_select(float if_clear, float if_set)
{
    constexpr uint64_t m = BIT == 4   ? 0xFFFF0000FFFF0000ull
                           : BIT == 3 ? 0xFF00FF00FF00FF00ull
                           : BIT == 2 ? 0xF0F0F0F0F0F0F0F0ull
                                      : 0xCCCCCCCCCCCCCCCCull;
    static_assert(BIT >= 1 && BIT <= 4, "lane bit");
    float r;
    asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(m));
    return r;
}

template <int BIT, int N> __device__ __forceinline__ void fold_half(float (&v)[16])
{
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float send = lane_bit_select<BIT>(v[k + N], v[k]);
        const float keep = lane_bit_select<BIT>(v[k], v[k + N]);
        v[k] = keep + lane_xor<1 << BIT>(send);
    }
}

// Sums each of 16 registers over the 32 lanes of a half-wave in 16 exchanges
// (not 16 x 5): lane p of the half returns the sum of register p >> 1.  The
// tree is fixed, so the result does not depend on timing.
__device__ __forceinline__ float half_wave_sum16(float (&v)[16])
{
    fold_half<4, 8>(v);
    fold_half<3, 4>(v);
    fold_half<2, 2>(v);
    fold_half<1, 1>(v);
    return v[0] + lane_xor<1>(v[0]);
}

// Activation statistics from the accumulators of one BM x BN output tile,
// taken before the packing (rows < M only):
//  * per (row, TwELL tile), the sum of the positive z: per lane, the positive
//    values of a group of min(TW, WN) columns are added in ascending block
//    order, the 32 lanes of each half-wave are reduced with half_wave_sum16,
//    and a tile wider than a wave adds its two waves' groups in column order;
//  * per column, the rows with z > 0: per lane over its rows, then the
//    2 x (BM / WM) lanes that share a column are added in LDS and go out with
//    one atomic add.
// The activity test is integer arithmetic on max(z, 0) in inline assembly,
// not a compare: the compiler turns any visible form of it back into a
// compare, merges that with the packing's ballots and keeps the masks live
// across both, spilling registers.  Uses the first BM * BN / 8 + (BM / WM) * BN * 8 bytes of smem;
// ends with a barrier.
template <int BM, int BN, int WM, int WN, int TW, int LDS_BYTES, bool PARTIAL>
__device__ __forceinline__ void gate_stats_tile(const f32x16 (&acc)[WM / 32][WN / 32], char *smem, int m0, int n0,
                                                int M, int N, int n_b, const GateStats &st)
{
    constexpr int FM = WM / 32, FN = WN / 32, NWN = BN / WN, NWM = BM / WM;
    constexpr int NTHR = NWM * NWN * 64;
    constexpr int GW = TW < WN ? TW : WN;  // columns of one row-sum group
    constexpr int GPW = WN / GW;           // groups per wave
    constexpr int FPG = GW / 32;           // accumulator blocks per group
    constexpr int GPR = BN / GW;           // groups per workgroup row
    constexpr int GPT = TW / GW;           // groups per TwELL tile (1 or 2)
    constexpr int TPW = BN / TW;           // TwELL tiles per workgroup row
    static_assert(GPT == 1 || GPT == 2, "a TwELL tile spans at most two waves");
    float *spart = reinterpret_cast<float *>(smem);                    // [BM][GPR]
    int32_t *scol = reinterpret_cast<int32_t *>(smem + BM * GPR * 4);  // [2 * NWM][BN]
    static_assert(BM * GPR * 4 + 2 * NWM * BN * 4 <= LDS_BYTES, "statistics LDS");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;
    const int rows_left = M - (m0 + wm * WM);  // rows of this wave below M

    int ccnt[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        ccnt[fn] = 0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int f = 0; f < FPG; ++f) {
                    // r = max(z, 0) (the accumulators hold no signalling NaN, and a
                    // quiet NaN gives 0); the count grows by 1 iff r is not +-0,
                    // i.e. z > 0 (and, PARTIAL, the row is below M).  The count is
                    // an in-out operand so each add happens here: deferred adds
                    // would keep every activity bit live.
                    float r;
                    uint32_t t;
                    if constexpr (PARTIAL) {
                        const uint32_t live = (uint32_t)(fm * 32 + acc_row(i, lane) - rows_left) >> 31;
                        asm("v_max_f32 %0, 0, %3\n\tv_lshlrev_b32 %1, 1, %0\n\tv_min_u32 %1, 1, %1\n\t"
                            "v_and_b32 %1, %1, %4\n\tv_add_u32 %2, %2, %1"
                            : "=&v"(r), "=&v"(t), "+v"(ccnt[g * FPG + f])
                            : "v"(acc[fm][g * FPG + f][i]), "v"(live));
                    } else {
                        asm("v_max_f32 %0, 0, %3\n\tv_lshlrev_b32 %1, 1, %0\n\tv_min_u32 %1, 1, %1\n\t"
                            "v_add_u32 %2, %2, %1"
                            : "=&v"(r), "=&v"(t), "+v"(ccnt[g * FPG + f])
                            : "v"(acc[fm][g * FPG + f][i]));
                    }
                    s += r;
                }
                v[i] = s;
            }
            const float r = half_wave_sum16(v);
            if (!(lane & 1)) {
                const int row = wm * WM + fm * 32 + acc_row((lane & 31) >> 1, lane);
                spart[row * GPR + wn * GPW + g] = r;
            }
        }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        scol[(wm * 2 + (lane >> 5)) * BN + wn * WN + fn * 32 + (lane & 31)] = ccnt[fn];
    __syncthreads();

    for (int e = tid; e < BM * TPW; e += NTHR) {
        const int r = e / TPW, tl = e - r * TPW;
        float s = spart[r * GPR + tl * GPT];
        if constexpr (GPT == 2)
            s += spart[r * GPR + tl * GPT + 1];
        const int t = m0 + r, gcol = n0 + tl * TW;
        if (t < M && gcol < N)
            st.l1[(int64_t)t * n_b + gcol / TW] = s;
    }
    for (int c = tid; c < BN; c += NTHR) {
        int s = 0;
#pragma unroll
        for (int j = 0; j < 2 * NWM; ++j)
            s += scol[j * BN + c];
        if (s && n0 + c < N)
            atomicAdd(st.neuron_cnt + n0 + c, s);
    }
    __syncthreads();
}

template <typename TI, int BM, int BN, int WM, int WN, int TW, int KB, int STAGES, int WPE, bool STATS>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
gate_twell_kernel(GemmArgs p, TwellOut<TI> o, GateStats st)
{
    using Core = GemmCore<TI, BM, BN, WM, WN, false, KB, STAGES>;
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    int mt, nt;
    tile_coords(blockIdx.x, p.MT, p.NT, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    Core core;
    f32x16 acc[Core::FM][Core::FN];
    core.run(p, smem, m0, n0, p.M, p.k_begin, p.k_len, threadIdx.x, acc);
    if constexpr (STATS) {
        if (m0 + BM <= p.M)
            gate_stats_tile<BM, BN, WM, WN, TW, Core::LDS_BYTES, false>(acc, smem, m0, n0, p.M, p.N, o.n_b, st);
        else
            gate_stats_tile<BM, BN, WM, WN, TW, Core::LDS_BYTES, true>(acc, smem, m0, n0, p.M, p.N, o.n_b, st);
    }
    if (seg_fits<TI, BM, BN, WN, TW, Core::LDS_BYTES>(o.cap))
        twell_epilogue_seg<TI, BM, BN, WM, WN, TW, Core::LDS_BYTES>(acc, smem, m0, n0, p.M, p.N, o);
    else
        twell_epilogue<TI, BM, BN, WM, WN, TW, Core::LDS_BYTES>(acc, smem, m0, n0, p.M, p.N, o);
}

// The same GEMM with a plain epilogue: h = ReLU(z) stored densely ([M][N],
// the storage type, round to nearest even), straight from the accumulators
// (a lane's 16 values of a 32 x 32 block are 16 rows of one column; the 32
// lanes of a half-wave write 64 or 128 contiguous bytes of each row).
template <typename TI, int BM, int BN, int WM, int WN, int KB, int STAGES, int WPE>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
gate_dense_kernel(GemmArgs p, TI *h)
{
    using Core = GemmCore<TI, BM, BN, WM, WN, false, KB, STAGES>;
    __shared__ __attribute__((aligned(16))) char smem[Core::LDS_BYTES];
    int mt, nt;
    tile_coords(blockIdx.x, p.MT, p.NT, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;
    Core core;
    f32x16 acc[Core::FM][Core::FN];
    core.run(p, smem, m0, n0, p.M, p.k_begin, p.k_len, threadIdx.x, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / Core::NWN, wn = wave % Core::NWN;
#pragma unroll
    for (int fm = 0; fm < Core::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Core::FN; ++fn)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm * WM + fm * 32 + acc_row(i, lane);
                const int n = n0 + wn * WN + fn * 32 + (lane & 31);
                if (m < p.M && n < p.N) {
                    const float v = acc[fm][fn][i];
                    store_elem(h + (int64_t)m * p.N + n, v > 0.f ? v : 0.f);
                }
            }
}

template <typename TI, int BM, int BN, int WM, int WN, int KB, int STAGES, int WPE>
static hipError_t gate_dense_go(const void *x, const void *wg_t, int T, int d, int F, void *h, hipStream_t s)
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
    constexpr int NTHR = (BM / WM) * (BN / WN) * 64;
    gate_dense_kernel<TI, BM, BN, WM, WN, KB, STAGES, WPE>
        <<<dim3(p.MT * p.NT), dim3(NTHR), 0, s>>>(p, static_cast<TI *>(h));
    return hipGetLastError();
}

hipError_t launch_gate_dense(int vdtype, const void *x, const void *wg_t, int T, int d, int F, void *h,
                             hipStream_t s)
{
    if (vdtype == 1)
        return gate_dense_go<__bf16, GATE_BM, 256, GATE_WM, 128, GATE_KB, GATE_STAGES, GATE_WPE>(x, wg_t, T, d, F,
                                                                                                 h, s);
    return gate_dense_go<float, 64, 256, 32, 128, 128, 2, 1>(x, wg_t, T, d, F, h, s);
}

template <typename TI, int BM, int BN, int WM, int WN, int KB, int STAGES, int WPE, bool STATS>
static hipError_t gate_twell_go(const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap, void *val,
                                uint8_t *idx, int32_t *cnt, const GateStats &st, hipStream_t s)
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
        gate_twell_kernel<TI, BM, BN, WM, WN, 32, KB, STAGES, WPE, STATS><<<grid, block, 0, s>>>(p, o, st);
        break;
    case 64:
        gate_twell_kernel<TI, BM, BN, WM, WN, 64, KB, STAGES, WPE, STATS><<<grid, block, 0, s>>>(p, o, st);
        break;
    case 128:
        gate_twell_kernel<TI, BM, BN, WM, WN, 128, KB, STAGES, WPE, STATS><<<grid, block, 0, s>>>(p, o, st);
        break;
    default:
        gate_twell_kernel<TI, BM, BN, WM, WN, 256, KB, STAGES, WPE, STATS><<<grid, block, 0, s>>>(p, o, st);
        break;
    }
    return hipGetLastError();
}

// Tile shapes: bf16 as configured above, fp32 64 x 256 (4 waves of 32 x 128).
template <bool STATS>
static hipError_t gate_twell_dispatch(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w,
                                      int cap, void *val, uint8_t *idx, int32_t *cnt, const GateStats &st,
                                      hipStream_t s)
{
    if (vdtype == 1)
        return gate_twell_go<__bf16, GATE_BM, 256, GATE_WM, 128, GATE_KB, GATE_STAGES, GATE_WPE, STATS>(
            x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, st, s);
    return gate_twell_go<float, 64, 256, 32, 128, 128, 2, 1, STATS>(x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, st,
                                                                    s);
}

hipError_t launch_gate_twell(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                             void *val, uint8_t *idx, int32_t *cnt, hipStream_t s)
{
    return gate_twell_dispatch<false>(vdtype, x, wg_t, T, d, F, tile_w, cap, val, idx, cnt, GateStats{}, s);
}

hipError_t launch_gate_twell_stats(int vdtype, const void *x, const void *wg_t, int T, int d, int F, int tile_w,
                                   int cap, void *val, uint8_t *idx, int32_t *cnt, int32_t *neuron_cnt, float *l1,
                                   hipStream_t s)
{
    return gate_twell_dispatch<true>(vdtype, x, wg_t, T, d, F, tile_w, cap, val, idx, cnt,
                                     GateStats{neuron_cnt, l1}, s);
}

}  // namespace twell
