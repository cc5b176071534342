// twell_device.h -- device-side building blocks of libtwell (gfx950 only).
//
// * 16-byte "chunk" loads and a swizzled LDS tile layout shared by every GEMM:
//   a tile row holds KB bytes of the K dimension (KB = 128: 64 bf16 / 32 fp32,
//   or KB = 64) as KB/16 chunks, XOR-swizzled per row (see lds_off) so that
//   16 consecutive rows read at one logical chunk hit 16 distinct 16-byte
//   bank groups, and a 1 KiB global->LDS copy (whole rows) does too.
// * MFMA step on one chunk per lane: bf16 -> one v_mfma_f32_32x32x16_bf16;
//   fp32 -> four v_mfma_f32_32x32x2f32.  Lanes 0-31 supply chunk 2s and lanes
//   32-63 chunk 2s+1 of the same rows; A and B use the same K mapping, so the
//   products are paired correctly whatever order the instruction sums them in.
// * 32x32 accumulator layout (16 floats per lane): element i of lane l is
//   row (i/4)*8 + (l/32)*4 + i%4, column l%32.  Hence one ballot over one
//   accumulator register yields two rows' 32-column activity masks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


namespace twell {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename TI> struct Elt;
template <> struct Elt<__bf16> {
    static constexpr int SIZE = 2;
    static constexpr int PER_CHUNK = 8;
};
template <> struct Elt<float> {
    static constexpr int SIZE = 4;
    static constexpr int PER_CHUNK = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Element e (0..PER_CHUNK-1) of a chunk, as fp32.
template <typename TI> __device__ __forceinline__ float chunk_elem(const u32x4 &c, int e);
template <> __device__ __forceinline__ float chunk_elem<__bf16>(const u32x4 &c, int e)
{
    uint32_t w = c[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}
template <> __device__ __forceinline__ float chunk_elem<float>(const u32x4 &c, int e) { return __uint_as_float(c[e]); }

// Store one value in the element type (bf16: round to nearest even).
__device__ __forceinline__ void store_elem(__bf16 *p, float v) { *p = (__bf16)v; }
__device__ __forceinline__ void store_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ float load_elem(const __bf16 *p) { return (float)*p; }
__device__ __forceinline__ float load_elem(const float *p) { return *p; }

__device__ __forceinline__ u32x4 ldg16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Byte offset of logical chunk `chunk` of tile row `row` in an LDS tile whose
// rows hold KB bytes (KB/16 chunks).  A 256-byte bank window holds 256/KB
// rows; the chunk slot is XORed with the row's index among the rows that share
// a window position, so 16 consecutive rows read at one logical chunk (one
// 16-lane phase of ds_read_b128) hit 16 distinct 16-byte bank groups.
template <int KB> __device__ __forceinline__ int lds_off(int row, int chunk)
{
    constexpr int CPR = KB / 16;        // chunks per row
    constexpr int RPW_LOG = KB == 128 ? 1 : 2;  // log2(rows per 256-byte window)
    return row * KB + ((chunk ^ ((row >> RPW_LOG) & (CPR - 1))) << 4);
}

__device__ __forceinline__ void mfma_chunk(__bf16, const u32x4 &a, const u32x4 &b, f32x16 &acc)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(float, const u32x4 &a, const u32x4 &b, f32x16 &acc)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int i, int lane) { return ((i >> 2) << 3) + ((lane >> 5) << 2) + (i & 3); }

// Output-tile placement.  Workgroups are handed to the 8 XCDs round-robin
// (workgroup g runs on XCD g % 8), each XCD with its own L2.  When the tile
// grid allows it, XCD x owns N-tile columns [x*NT/8, (x+1)*NT/8), walked in
// groups of 8 M-tiles, so the workgroups an XCD runs together share a few A
// and B tiles in its L2.
__device__ __forceinline__ void tile_coords(int g, int MT, int NT, int &mt, int &nt)
{
    if ((NT & 7) == 0 && MT * NT >= 64) {
        const int xcd = g & 7, s = g >> 3;
        const int ncol = NT >> 3;
        const int per_group = 8 * ncol;
        const int grp = s / per_group, r = s - grp * per_group;
        const int rem = MT - grp * 8;
        const int mrows = rem < 8 ? rem : 8;
        mt = grp * 8 + r % mrows;
        nt = xcd * ncol + r / mrows;
    } else {
        mt = g % MT;
        nt = g / MT;
    }
}

// ------------------------------------------------------------------ GEMM core
// C[m][n] = sum_k A[m][k] * B(k, n) over k in [k_begin, k_begin + k_len).
// A rows are K-contiguous (optionally gathered through a_rows).  B is either
// "NK" (B^T stored [N][K], K-contiguous: W_g^T, W_u^T) or "KN" ([K][N],
// N-contiguous: W_d), the latter read from its raw rows with transposing LDS
// reads (bf16) or transposed inside LDS stage by stage (fp32).
// Dual NK mode (block size DB > 0): two B matrices of the same shape (B, B2)
// share the A tile; the B tile's rows alternate between them in blocks of DB
// (rows 2 DB q + r, r < DB, are B's column DB q + r; rows 2 DB q + DB + r are
// B2's), so a wave whose tile is 2 DB rows wide holds both products of the
// same DB columns.
struct GemmArgs {
    const void *A;
    int64_t lda;             // elements
    const int32_t *a_rows;   // optional gather: A row of output row m is a_rows[m]
    int M;                   // rows of the output (upper bound)
    const int32_t *m_count;  // optional device count: rows used = min(*m_count, M)
    const void *B;
    int64_t ldb;             // elements
    int N;
    int k_begin, k_len;      // elements; k_len multiple of the 128-byte K tile
    int k_split_len;         // split-K: workgroup z-slice s covers [k_begin + s*k_split_len, +k_split_len)
    int MT, NT;              // tile grid
    uint32_t a_bytes, b_bytes;  // extents of A and B (each below 4 GiB)
    const void *B2;          // dual mode: second B, same ldb and extent as B
};

// Buffer resource over one matrix (raw, stride 0): word 3 as CDNA3/CDNA4
// expect for untyped dword loads.  `bytes` is the extent of the matrix.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes LDS bytes [dst + 16 l, dst + 16 l + 16).  No VGPRs hold the data.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *dst, int voff, int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

// Workgroup barrier without the release/acquire fence of __syncthreads(): that
// fence makes the compiler wait for every outstanding global->LDS copy
// (vmcnt(0)) before the barrier, which would drain a multi-stage copy ring at
// each stage.  Callers wait for exactly what must be complete with their own
// s_waitcnt first; the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename TI, int BM, int BN, int WM, int WN, bool B_KN, int KB = 128, int STAGES = 2, int DUALB = 0>
struct GemmCore {
    static constexpr int NWM = BM / WM, NWN = BN / WN;
    static constexpr int NW = NWM * NWN;
    static constexpr int NTHR = NW * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int E = Elt<TI>::PER_CHUNK;
    static constexpr int SZ = Elt<TI>::SIZE;
    static constexpr int CPR = KB / 16;                  // chunks per operand tile row
    static constexpr int KT = KB / SZ;                   // K elements per stage
    static constexpr int SUB = KB / 32;                  // MFMA sub-steps per stage
    static constexpr int RPC = 1024 / KB;                // operand tile rows per 1 KiB copy
    static constexpr int LDS_A = BM * KB, LDS_B = BN * KB;
    // K-contiguous ("NK") operands arrive by global->LDS copies of 1 KiB per
    // wave instruction (RPC whole operand rows).  A KN-layout B ([K][N],
    // N-contiguous) arrives the same way as raw [KT][BN] rows.  bf16 (B_TR):
    // the MFMA fragments are read from the raw rows with gfx950's transposing
    // LDS reads (ds_read_b64_tr_b16), the raw rows' 16-byte chunks XOR-swizzled
    // on the copy side.  fp32: the stage is transposed inside LDS, 4 x 4
    // blocks at a time, into the operand layout before the stage's MFMAs.
    static constexpr bool B_TR = B_KN && SZ == 2;
    static constexpr int RAW_ROW = BN * SZ;              // bytes of one raw B row
    static constexpr int B_RAW = B_KN ? KT * RAW_ROW : 0;
    static constexpr int RAW_RPI = B_KN ? 1024 / RAW_ROW : 1;  // raw rows per 1 KiB copy
    static constexpr int A_LD = BM / RPC / NW;
    static constexpr int B_LD = B_KN ? KT / RAW_RPI / NW : BN / RPC / NW;
    static constexpr int B_UNITS = B_KN ? (KT / E) * (BN / E) : 0;  // transpose blocks per stage
    static constexpr int BUF = LDS_A + (B_KN ? B_RAW : LDS_B);       // one ring slot
    static constexpr int LDS_BYTES = STAGES * BUF + (B_KN && !B_TR ? LDS_B : 0);
    static_assert(KB == 64 || KB == 128, "stage row width");
    static_assert(STAGES >= 2 && STAGES <= 8, "pipeline depth");
    static_assert((BM / RPC) % NW == 0, "A tile rows split over the waves");
    static_assert(B_KN || (BN / RPC) % NW == 0, "B tile rows split over the waves");
    static_assert(!B_KN || (1024 % RAW_ROW == 0 && (KT / RAW_RPI) % NW == 0), "raw B rows split over the waves");
    static_assert(!B_KN || B_UNITS % NTHR == 0 || B_UNITS < NTHR, "transpose blocks split over the threads");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is whole 32x32 blocks");
    static_assert(!B_KN || KB == 128, "the transposed B tile's swizzle assumes 128-byte rows");
    static_assert(!B_TR || (RAW_ROW % 256 == 0 && WN % 32 == 0), "raw rows span whole 256-byte bank windows");
    static_assert(DUALB == 0 || (!B_KN && BN % (2 * DUALB) == 0 && WN == 2 * DUALB && DUALB % RPC == 0),
                  "dual B: DUALB-row blocks, each wave spans one block of each matrix");

    // LDS byte offset of (row, 16-byte chunk) in the B operand tile.  NK: the
    // copy layout.  KN, fp32 (written by transpose_b): the chunk is XOR-ed with bits
    // 1-3 of the row and bits 4-6, so that both the fragment reads (16
    // consecutive rows) and the transposing stores (rows 8 apart, both
    // parities) of a 16-lane phase hit 16 distinct 16-byte bank groups.
    __device__ __forceinline__ static int b_off(int row, int chunk)
    {
        if constexpr (B_KN)
            return row * KB + ((chunk ^ (((row >> 1) ^ (row >> 4)) & 7)) << 4);
        else
            return lds_off<KB>(row, chunk);
    }

    // B_TR: chunk slot of logical 16-byte chunk c in raw row r.  Rows k..k+3
    // (k a multiple of 4) put any 4 consecutive chunks of a 256-byte window on
    // 16 distinct slots, so the 32 lanes of a transposing read (4 rows x 64
    // bytes) hit every bank once.
    __device__ __forceinline__ static int raw_slot(int r, int c) { return c ^ ((r & 3) << 2); }

    __amdgpu_buffer_rsrc_t ra, rb, rb2;
    int a_voff[A_LD];
    int b_voff[B_LD > 0 ? B_LD : 1];
    int wave;
    int b_stage_bytes;  // KN: bytes of K rows per stage in global memory

    // Copy j of this wave fills operand rows g*RPC + l/CPR (g = j*NW + wave) at
    // physical chunk slot l%CPR, i.e. it loads the logical chunk the swizzle
    // maps there.  KN raw copies fill raw rows g*RAW_RPI + l/(RAW_ROW/16).
    __device__ __forceinline__ void setup(const GemmArgs &p, int m0, int n0, int m_used, int kb, int tid)
    {
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
        const int lane = tid & 63;
        constexpr int RPW_LOG = KB == 128 ? 1 : 2;
        ra = make_rsrc(p.A, p.a_bytes);
        rb = make_rsrc(p.B, p.b_bytes);
        if constexpr (DUALB > 0)
            rb2 = make_rsrc(p.B2, p.b_bytes);
#pragma unroll
        for (int j = 0; j < A_LD; ++j) {
            const int r = (j * NW + wave) * RPC + lane / CPR;
            const int c = (lane % CPR) ^ ((r >> RPW_LOG) & (CPR - 1));
            int gm = m0 + r;
            gm = gm < m_used ? gm : m_used - 1;  // rows past the end re-read a valid row; results discarded
            const int64_t ar = p.a_rows ? (int64_t)p.a_rows[gm] : (int64_t)gm;
            a_voff[j] = (int)((ar * p.lda + kb) * SZ + c * 16);
        }
        if constexpr (!B_KN) {
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                const int r = (j * NW + wave) * RPC + lane / CPR;
                const int c = (lane % CPR) ^ ((r >> RPW_LOG) & (CPR - 1));
                int gn = DUALB > 0 ? n0 + r / (2 * DUALB) * DUALB + r % DUALB : n0 + r;
                gn = gn < p.N ? gn : p.N - 1;
                b_voff[j] = (int)(((int64_t)gn * p.ldb + kb) * SZ + c * 16);
            }
        } else {
            constexpr int LPR = RAW_ROW / 16;  // lanes per raw row
            b_stage_bytes = KT * (int)p.ldb * SZ;
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                const int r = (j * NW + wave) * RAW_RPI + lane / LPR;  // k row within the stage
                // the copy writes slot lane % LPR of the row: load the chunk that belongs there
                const int c = B_TR ? raw_slot(r, lane % LPR) : lane % LPR;
                int gn = n0 + c * E;
                gn = gn <= p.N - E ? gn : p.N - E;  // columns past N re-read valid ones; results discarded
                b_voff[j] = (int)(((int64_t)(kb + r) * p.ldb + gn) * SZ);
            }
        }
    }

    // Copy c of stage kt's A_LD + B_LD copies (A first) into ring slot `buf`.
    __device__ __forceinline__ void load_one(int kt, char *buf, int c)
    {
        const int koff = kt * KB;
        if (c < A_LD) {
            dma16(ra, buf + (c * NW + wave) * 1024, a_voff[c], koff);
        } else {
            const int j = c - A_LD;
            dma16(rb, buf + LDS_A + (j * NW + wave) * 1024, b_voff[j], koff);
        }
    }

    // One MFMA sub-step with copies C0..C1-1 of stage kt spread evenly
    // between its MFMAs (kept in that order), so the copy queue fills at the
    // rate it drains instead of all at once.
    // `on` (wave-uniform) only gates the copies: the MFMAs run on every path,
    // so the accumulators never merge from two versions.
    template <int C0, int C1>
    __device__ __forceinline__ void mfma_sub_copies(const u32x4 (&af)[FM], const u32x4 (&bf)[FN],
                                                    f32x16 (&acc)[FM][FN], int kt, char *buf, bool on)
    {
        constexpr int NM = FM * FN, NC = C1 - C0;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            mfma_chunk(TI{}, af[q / FN], bf[q % FN], acc[q / FN][q % FN]);
#pragma unroll
            for (int c = C0; c < C1; ++c)
                if ((c - C0) * NM / NC == q && on)
                    load_one(kt, buf, c);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Queue stage kt's global->LDS copies into ring slot `buf`.
    __device__ __forceinline__ void load(int kt, char *buf)
    {
        char *sa = buf, *sb = buf + LDS_A;
        const int koff = kt * KB;
#pragma unroll
        for (int j = 0; j < A_LD; ++j)
            dma16(ra, sa + (j * NW + wave) * 1024, a_voff[j], koff);
        if constexpr (DUALB > 0) {
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                // the copy's RPC rows lie in one DUALB-row block, whose parity picks the matrix
                if ((((j * NW + wave) * RPC) / DUALB) & 1)
                    dma16(rb2, sb + (j * NW + wave) * 1024, b_voff[j], koff);
                else
                    dma16(rb, sb + (j * NW + wave) * 1024, b_voff[j], koff);
            }
        } else if constexpr (!B_KN) {
#pragma unroll
            for (int j = 0; j < B_LD; ++j)
                dma16(rb, sb + (j * NW + wave) * 1024, b_voff[j], koff);
        } else {
            const int boff = (int)((uint32_t)kt * (uint32_t)b_stage_bytes);
#pragma unroll
            for (int j = 0; j < B_LD; ++j)
                dma16(rb, sb + (j * NW + wave) * 1024, b_voff[j], boff);
        }
    }

    // KN, fp32: raw [KT][BN] rows of slot `buf` -> operand layout in `bop`.
    // Thread u handles the E x E block at k-group u / (BN/E), n-group u % (BN/E).
    __device__ __forceinline__ void transpose_b(const char *buf, char *bop, int tid)
    {
        if constexpr (B_KN && !B_TR) {
            const char *raw = buf + LDS_A;
#pragma unroll
            for (int u0 = 0; u0 < B_UNITS; u0 += NTHR) {
                const int u = u0 + tid;
                if (B_UNITS < NTHR && u >= B_UNITS)
                    break;
                const int ng = u % (BN / E), kg = u / (BN / E);
                u32x4 rr[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    rr[e] = *reinterpret_cast<const u32x4 *>(raw + (kg * E + e) * RAW_ROW + ng * 16);
                u32x4 o[E];  // o[n]: column n of the block, its E k values
#pragma unroll
                for (int n = 0; n < E; ++n)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        o[n][w] = rr[w][n];
                // Odd n-groups write their columns in the order 1, 0, 3, 2, ...:
                // each store then covers rows of both parities, which with the
                // B-tile swizzle puts every 16-lane phase on 16 distinct bank groups.
                const int odd = ng & 1;
                const uint32_t msk = 0u - (uint32_t)odd;  // all ones for an odd n-group
#pragma unroll
                for (int q = 0; q < E; ++q) {
                    u32x4 w;  // o[q ^ odd], as a bit blend (an indexed pick compiles to a select chain)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w[i] = o[q][i] ^ ((o[q][i] ^ o[q ^ 1][i]) & msk);
                    *reinterpret_cast<u32x4 *>(bop + b_off(ng * E + (q ^ odd), kg)) = w;
                }
            }
        }
    }

    // The MFMA sub-steps of one stage; fragments of sub-step s+1 are read from
    // LDS while the MFMAs of sub-step s run.
    __device__ __forceinline__ void compute(const char *sa, const char *sb, int wm, int wn, int lane,
                                            f32x16 (&acc)[FM][FN])
    {
        const int lr = lane & 31, lh = lane >> 5;
        u32x4 af[2][FM], bfr[2][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            af[0][fm] = *reinterpret_cast<const u32x4 *>(sa + lds_off<KB>(wm * WM + fm * 32 + lr, lh));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            bfr[0][fn] = *reinterpret_cast<const u32x4 *>(sb + b_off(wn * WN + fn * 32 + lr, lh));
#pragma unroll
        for (int ss = 0; ss < SUB; ++ss) {
            const int cb = ss & 1, nb = cb ^ 1;
            if (ss + 1 < SUB) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    af[nb][fm] = *reinterpret_cast<const u32x4 *>(
                        sa + lds_off<KB>(wm * WM + fm * 32 + lr, (ss + 1) * 2 + lh));
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    bfr[nb][fn] = *reinterpret_cast<const u32x4 *>(
                        sb + b_off(wn * WN + fn * 32 + lr, (ss + 1) * 2 + lh));
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    mfma_chunk(TI{}, af[cb][fm], bfr[cb][fn], acc[fm][fn]);
        }
        // nothing of this stage may sink below the wait for the next stage's copies
        __builtin_amdgcn_sched_barrier(0);
    }

    // Wait for this wave's copies of stage kt when `ahead` later stages were
    // queued after it (their copies may stay in flight).  Also drains LDS ops.
    template <int AHEAD> __device__ __forceinline__ static void wait_n()
    {
        constexpr int PER = A_LD + B_LD;
        constexpr int V = AHEAD * PER;
        static_assert(V <= 63, "vmcnt range");
        __builtin_amdgcn_s_waitcnt(0x0070 | (V & 15) | ((V >> 4) << 14));
    }
    template <int N> __device__ __forceinline__ static void wait_upto(int ahead)
    {
        if constexpr (N == 0) {
            wait_n<0>();
        } else {
            if (ahead >= N)
                wait_n<N>();
            else
                wait_upto<N - 1>(ahead);
        }
    }
    __device__ __forceinline__ void wait_stage(int ahead) { wait_upto<STAGES - 2>(ahead); }

    // Fragments of MFMA sub-step ss (16 bf16 / 4 fp32 K elements) from a slot.
    __device__ __forceinline__ void read_frags(const char *sa, const char *sb, int wm, int wn, int lane, int ss,
                                               u32x4 (&af)[FM], u32x4 (&bf)[FN])
    {
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            af[fm] = *reinterpret_cast<const u32x4 *>(sa + lds_off<KB>(wm * WM + fm * 32 + lr, ss * 2 + lh));
        if constexpr (B_TR) {
            // Lane l needs B(k0 + e, n) for e < 8, n = its column (l % 32), k0 =
            // 16 ss + 8 (l / 32): the same K chunk as its A fragment.  Within a
            // 16-lane group the transposing read hands lane i element i % 4 of
            // the 8-byte pieces addressed by lanes i / 4 + 4 j (j < 4) as its
            // values j: so lane p addresses row k0 + p / 4 (+ 4 for the second
            // half), columns 4 (p % 4) .. +3 of the group's 16.
            const int g = lane >> 4, pp = lane & 15;
            const int kr = ss * 16 + ((g >> 1) << 3) + (pp >> 2);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = wn * WN + fn * 32 + ((g & 1) << 4) + ((pp & 3) << 2);
                typedef short v4s __attribute__((ext_vector_type(4)));
                v4s h[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int r = kr + 4 * half;
                    const char *pa = sb + r * RAW_ROW + (raw_slot(r, n >> 3) << 4) + (((n >> 2) & 1) << 3);
                    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(pa));
                }
                bf[fn] = u32x4{(uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16),
                               (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16),
                               (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16),
                               (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16)};
            }
        } else {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf[fn] = *reinterpret_cast<const u32x4 *>(sb + b_off(wn * WN + fn * 32 + lr, ss * 2 + lh));
        }
    }
    __device__ __forceinline__ static void mfma_sub(const u32x4 (&af)[FM], const u32x4 (&bf)[FN],
                                                    f32x16 (&acc)[FM][FN])
    {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                mfma_chunk(TI{}, af[fm], bf[fn], acc[fm][fn]);
    }

    // K loop for NK operands, pipelined across stages: the wait and barrier
    // for stage kt+1 come before the MFMAs of stage kt's last sub-step, so the
    // first fragment reads of kt+1 overlap those MFMAs instead of following a
    // barrier with the MFMA pipe idle.  Past that barrier every wave holds the
    // rest of stage kt in registers, so the copy for stage kt+STAGES goes into
    // stage kt's slot.  Ends with a barrier so the caller may reuse `smem`.
    __device__ __forceinline__ void run_nk(const GemmArgs &p, char *smem, int m0, int n0, int m_used, int kb,
                                           int klen, int tid, f32x16 (&acc)[FM][FN])
    {
        static_assert((!B_KN || B_TR) && SUB % 2 == 0, "fragment buffers alternate within a stage");
        const int lane = tid & 63;
        const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wv / NWN, wn = wv % NWN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[fm][fn][i] = 0.f;
        setup(p, m0, n0, m_used, kb, tid);
        const int nk = klen / KT;
        if (nk > 0) {
#pragma unroll
            for (int s = 0; s < STAGES - 1; ++s)
                if (s < nk)
                    load(s, smem + s * BUF);
            wait_stage(nk - 1 < STAGES - 2 ? nk - 1 : STAGES - 2);
            wg_barrier();
            u32x4 af[2][FM], bf[2][FN];
            read_frags(smem, smem + LDS_A, wm, wn, lane, 0, af[0], bf[0]);
            if (STAGES - 1 < nk)
                load(STAGES - 1, smem + (STAGES - 1) * BUF);
            int slot = 0;  // ring slot of stage kt (= kt % STAGES)
            for (int kt = 0; kt < nk; ++kt) {
                char *cur = smem + slot * BUF;
                const int nslot = slot + 1 == STAGES ? 0 : slot + 1;
#pragma unroll
                for (int ss = 0; ss < SUB; ++ss) {
                    const int cb = ss & 1, nb = cb ^ 1;
                    if (ss + 1 < SUB) {
                        read_frags(cur, cur + LDS_A, wm, wn, lane, ss + 1, af[nb], bf[nb]);
                        // issued before this sub-step's MFMAs, not after them: left alone
                        // the scheduler gives them the registers those MFMAs free
                        __builtin_amdgcn_sched_barrier(0);
                    } else {
                        // earlier sub-steps' MFMAs stay above the waits
                        __builtin_amdgcn_sched_barrier(0);
                        // this stage's last fragments have arrived (on every path, so the
                        // compiler adds no partial waits before the MFMAs below)
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    }
                    if (ss + 1 == SUB && kt + 1 < nk) {
                        const int left = nk - 2 - kt;  // stages queued after kt+1
                        wait_stage(left < STAGES - 2 ? left : STAGES - 2);
                        wg_barrier();
                        const char *nxt = smem + nslot * BUF;
                        read_frags(nxt, nxt + LDS_A, wm, wn, lane, 0, af[nb], bf[nb]);
                        if (kt + STAGES < nk)
                            load(kt + STAGES, cur);
                    }
                    mfma_sub(af[cb], bf[cb], acc);
                }
                slot = nslot;
            }
        }
        __syncthreads();
    }

    // K loop for NK operands, 2-slot ring, copies spread over the MFMAs: the
    // copies of stage kt + 2 (into stage kt's slot, free once the barrier
    // before stage kt's last sub-step has passed) are issued in two halves,
    // between the MFMAs of that last sub-step and of stage kt + 1's first.
    // The barrier before stage kt + 2 waits for all of them (vmcnt(0)).
    __device__ __forceinline__ void run_nk_spread(const GemmArgs &p, char *smem, int m0, int n0, int m_used, int kb,
                                                  int klen, int tid, f32x16 (&acc)[FM][FN])
    {
        static_assert(STAGES == 2 && !B_KN && DUALB == 0 && SUB % 2 == 0, "spread copies: NK, 2 slots");
        constexpr int NC = A_LD + B_LD, H = NC / 2;
        const int lane = tid & 63;
        const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wv / NWN, wn = wv % NWN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[fm][fn][i] = 0.f;
        setup(p, m0, n0, m_used, kb, tid);
        const int nk = klen / KT;
        if (nk > 0) {
            load(0, smem);
            wait_n<0>();
            wg_barrier();
            u32x4 af[2][FM], bf[2][FN];
            read_frags(smem, smem + LDS_A, wm, wn, lane, 0, af[0], bf[0]);
            if (nk > 1)
                load(1, smem + BUF);
            int slot = 0;
#pragma clang loop unroll(disable)
            for (int kt = 0; kt < nk; ++kt) {
                char *cur = smem + slot * BUF;
                const int nslot = slot ^ 1;
                // the second half of stage kt + 1's copies (first half queued during stage kt - 1)
                const bool pend = kt >= 1 && kt + 1 < nk;
#pragma unroll
                for (int ss = 0; ss < SUB; ++ss) {
                    const int cb = ss & 1, nb = cb ^ 1;
                    if (ss + 1 < SUB) {
                        read_frags(cur, cur + LDS_A, wm, wn, lane, ss + 1, af[nb], bf[nb]);
                        __builtin_amdgcn_sched_barrier(0);
                    } else {
                        __builtin_amdgcn_sched_barrier(0);
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    }
                    if (ss + 1 == SUB) {
                        if (kt + 1 < nk) {
                            wait_n<0>();
                            wg_barrier();
                            const char *nxt = smem + nslot * BUF;
                            read_frags(nxt, nxt + LDS_A, wm, wn, lane, 0, af[nb], bf[nb]);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        mfma_sub_copies<0, H>(af[cb], bf[cb], acc, kt + 2, cur, kt + 2 < nk);
                    } else if (ss == 0) {
                        mfma_sub_copies<H, NC>(af[cb], bf[cb], acc, kt + 1, smem + nslot * BUF, pend);
                    } else {
                        mfma_sub(af[cb], bf[cb], acc);
                    }
                }
                slot = nslot;
            }
        }
        __syncthreads();
    }

    // Full K loop.  NK operands, 2-slot ring (the gate): run_nk_spread; other
    // NK rings and transposing-read KN (bf16): run_nk.  KN B: an STAGES-deep ring of LDS
    // slots fed by global->LDS copies issued STAGES-1 stages ahead, two
    // barriers per stage (the stage is transposed in LDS first).  Ends with a
    // barrier so the caller may reuse `smem`.
    __device__ __forceinline__ void run(const GemmArgs &p, char *smem, int m0, int n0, int m_used, int kb, int klen,
                                        int tid, f32x16 (&acc)[FM][FN])
    {
        if constexpr (STAGES == 2 && !B_KN && DUALB == 0 && SUB % 2 == 0) {
            run_nk_spread(p, smem, m0, n0, m_used, kb, klen, tid, acc);
            return;
        } else if constexpr (!B_KN || B_TR) {
            run_nk(p, smem, m0, n0, m_used, kb, klen, tid, acc);
            return;
        }
        const int lane = tid & 63;
        const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wv / NWN, wn = wv % NWN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[fm][fn][i] = 0.f;
        setup(p, m0, n0, m_used, kb, tid);
        const int nk = klen / KT;
        char *bop = smem + STAGES * BUF;  // KN operand tile
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nk)
                load(s, smem + s * BUF);
        int slot = 0;  // ring slot of stage kt
        for (int kt = 0; kt < nk; ++kt) {
            const int left = nk - 1 - kt;  // stages queued after kt
            wait_stage(left < STAGES - 2 ? left : STAGES - 2);
            wg_barrier();
            char *cur = smem + slot * BUF;
            if constexpr (B_KN) {
                transpose_b(cur, bop, tid);
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                wg_barrier();
            }
            if (kt + STAGES - 1 < nk) {
                int ls = slot + STAGES - 1;
                ls = ls >= STAGES ? ls - STAGES : ls;
                load(kt + STAGES - 1, smem + ls * BUF);
            }
            compute(cur, B_KN ? bop : cur + LDS_A, wm, wn, lane, acc);
            slot = slot + 1 == STAGES ? 0 : slot + 1;
        }
        __syncthreads();
    }
};

}  // namespace twell
