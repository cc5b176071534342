// twell_device.h -- device-side building blocks of libtwell (gfx950 only).
//
// * 16-byte "chunk" loads and a swizzled LDS tile layout shared by every GEMM:
//   a tile row holds 128 bytes of the K dimension (64 bf16 or 32 fp32) as 8
//   chunks; chunk c of row r lives at chunk slot c ^ (r & 7), so the 32 rows a
//   half-wave reads for one MFMA operand hit 8 distinct 16-byte bank groups.
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
__device__ __forceinline__ float round_to_elem(__bf16, float v) { return (float)(__bf16)v; }
__device__ __forceinline__ float round_to_elem(float, float v) { return v; }

__device__ __forceinline__ u32x4 ldg16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ int lds_off(int row, int chunk) { return (row << 7) + ((chunk ^ (row & 7)) << 4); }

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
// N-contiguous: W_d), the latter transposed in registers on its way to LDS.
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
};

template <typename TI, int BM, int BN, int WM, int WN, bool B_KN>
struct GemmCore {
    static constexpr int NWM = BM / WM, NWN = BN / WN;
    static constexpr int NTHR = NWM * NWN * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int E = Elt<TI>::PER_CHUNK;
    static constexpr int KT = 128 / Elt<TI>::SIZE;      // K elements per tile
    static constexpr int A_CH = BM * 8 / NTHR;          // A chunks per thread per tile
    static constexpr int B_CH = B_KN ? 0 : BN * 8 / NTHR;
    static constexpr int B_UNITS = B_KN ? 8 * BN / E : 0;  // E x E transpose units per tile
    static constexpr int B_UPT = B_KN ? (B_UNITS + NTHR - 1) / NTHR : 0;
    static constexpr int LDS_A = BM * 128, LDS_B = BN * 128;
    static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B);
    static_assert(BM * 8 % NTHR == 0, "A tile load split");
    static_assert(B_KN || (BN * 8 % NTHR == 0), "B tile load split");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is whole 32x32 blocks");

    const char *a_ptr[A_CH];
    int a_lds[A_CH];
    const char *b_ptr[B_KN ? 1 : B_CH];
    int b_lds[B_KN ? 1 : B_CH];
    u32x4 a_reg[A_CH];
    u32x4 b_reg[B_KN ? (B_UPT * E) : B_CH];
    const char *bkn_ptr[B_KN ? B_UPT : 1];
    int bkn_row0[B_KN ? B_UPT : 1], bkn_chunk[B_KN ? B_UPT : 1];
    bool bkn_on[B_KN ? B_UPT : 1];
    int64_t ldb_bytes;

    __device__ __forceinline__ void setup(const GemmArgs &p, int m0, int n0, int m_used, int kb, int tid)
    {
        constexpr int SZ = Elt<TI>::SIZE;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int q = tid + i * NTHR;
            const int r = q >> 3, c = q & 7;
            int gm = m0 + r;
            gm = gm < m_used ? gm : m_used - 1;  // rows past the end read a valid row; results discarded
            const int64_t ar = p.a_rows ? (int64_t)p.a_rows[gm] : (int64_t)gm;
            a_ptr[i] = (const char *)p.A + (ar * p.lda + kb) * SZ + c * 16;
            a_lds[i] = lds_off(r, c);
        }
        if constexpr (!B_KN) {
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const int q = tid + i * NTHR;
                const int r = q >> 3, c = q & 7;
                int gn = n0 + r;
                gn = gn < p.N ? gn : p.N - 1;
                b_ptr[i] = (const char *)p.B + ((int64_t)gn * p.ldb + kb) * SZ + c * 16;
                b_lds[i] = lds_off(r, c);
            }
        } else {
            ldb_bytes = p.ldb * SZ;
#pragma unroll
            for (int i = 0; i < B_UPT; ++i) {
                const int u = tid + i * NTHR;
                bkn_on[i] = u < B_UNITS;
                const int kg = u & 7, ng = u >> 3;  // k group (chunk within the K tile), n group
                int gn = n0 + ng * E;
                gn = gn <= p.N - E ? gn : p.N - E;
                bkn_ptr[i] = (const char *)p.B + ((int64_t)(kb + kg * E) * p.ldb + gn) * SZ;
                bkn_row0[i] = ng * E;
                bkn_chunk[i] = kg;
            }
        }
    }

    __device__ __forceinline__ void load(int kt)
    {
        const int64_t koff = (int64_t)kt * 128;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            a_reg[i] = ldg16(a_ptr[i] + koff);
        if constexpr (!B_KN) {
#pragma unroll
            for (int i = 0; i < B_CH; ++i)
                b_reg[i] = ldg16(b_ptr[i] + koff);
        } else {
            const int64_t krow = (int64_t)kt * KT * ldb_bytes;
#pragma unroll
            for (int i = 0; i < B_UPT; ++i)
                if (bkn_on[i]) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        b_reg[i * E + e] = ldg16(bkn_ptr[i] + krow + e * ldb_bytes);
                }
        }
    }

    __device__ __forceinline__ void store(char *sa, char *sb)
    {
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            *reinterpret_cast<u32x4 *>(sa + a_lds[i]) = a_reg[i];
        if constexpr (!B_KN) {
#pragma unroll
            for (int i = 0; i < B_CH; ++i)
                *reinterpret_cast<u32x4 *>(sb + b_lds[i]) = b_reg[i];
        } else {
#pragma unroll
            for (int i = 0; i < B_UPT; ++i)
                if (bkn_on[i]) {
                    // b_reg[i*E + e] holds row k = e, columns n = 0..E-1; LDS wants, for
                    // each column n, the E k-values as one chunk.
#pragma unroll
                    for (int n = 0; n < E; ++n) {
                        u32x4 o;
                        if constexpr (Elt<TI>::SIZE == 2) {
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                const uint32_t lo = b_reg[i * E + 2 * w][n >> 1];
                                const uint32_t hi = b_reg[i * E + 2 * w + 1][n >> 1];
                                const uint32_t l16 = (n & 1) ? (lo >> 16) : (lo & 0xFFFFu);
                                const uint32_t h16 = (n & 1) ? (hi >> 16) : (hi & 0xFFFFu);
                                o[w] = l16 | (h16 << 16);
                            }
                        } else {
#pragma unroll
                            for (int w = 0; w < 4; ++w)
                                o[w] = b_reg[i * E + w][n];
                        }
                        *reinterpret_cast<u32x4 *>(sb + lds_off(bkn_row0[i] + n, bkn_chunk[i])) = o;
                    }
                }
        }
    }

    __device__ __forceinline__ void compute(const char *sa, const char *sb, int wm, int wn, int lane,
                                            f32x16 (&acc)[FM][FN])
    {
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
            u32x4 af[FM], bfr[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[fm] = *reinterpret_cast<const u32x4 *>(sa + lds_off(wm * WM + fm * 32 + lr, ss * 2 + lh));
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bfr[fn] = *reinterpret_cast<const u32x4 *>(sb + lds_off(wn * WN + fn * 32 + lr, ss * 2 + lh));
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    mfma_chunk(TI{}, af[fm], bfr[fn], acc[fm][fn]);
        }
    }

    // Full K loop with a double-buffered LDS tile; ends with a barrier so the
    // caller may reuse `smem`.
    __device__ __forceinline__ void run(const GemmArgs &p, char *smem, int m0, int n0, int m_used, int kb,
                                        int klen, int tid, f32x16 (&acc)[FM][FN])
    {
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / NWN, wn = wave % NWN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[fm][fn][i] = 0.f;
        setup(p, m0, n0, m_used, kb, tid);
        const int nk = klen / KT;
        constexpr int BUF = LDS_A + LDS_B;
        load(0);
        store(smem, smem + LDS_A);
        __syncthreads();
        for (int kt = 0; kt + 1 < nk; ++kt) {
            char *cur = smem + (kt & 1) * BUF;
            char *nxt = smem + ((kt + 1) & 1) * BUF;
            load(kt + 1);
            compute(cur, cur + LDS_A, wm, wn, lane, acc);
            store(nxt, nxt + LDS_A);
            __syncthreads();
        }
        char *last = smem + ((nk - 1) & 1) * BUF;
        compute(last, last + LDS_A, wm, wn, lane, acc);
        __syncthreads();
    }
};

}  // namespace twell
