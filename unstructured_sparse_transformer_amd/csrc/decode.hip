// decode.hip -- gate and TwELL packing for decode-shaped calls (T <= 64).
//
// "Sparser, Faster, Lighter Transformer Language Models" (gist.science
// summary), sections 2.1-2.3: the same gate, TwELL packing and overflow
// partition as the batch path, organised for a handful of tokens.  With
// T <= 64 the gate is a skinny GEMM bound by reading W_g once (d x F bf16);
// the batch kernel's 256 x 256 tiles would give only F / 256 workgroups, so
// here every workgroup owns 32 neurons (F / 32 workgroups) and its 8 waves
// split the K dimension.  Two organisations of the rest:
// * T <= 16 (gate_gather_kernel, reduce_pack_kernel): each gate workgroup
//   gathers its own 32 neurons' W_u / W_d rows right after its gate values
//   and writes one partial y row per row with an active neuron among them;
//   the second kernel adds those in a fixed order while it packs TwELL.
// * larger T, and the allocation-free call (gate_skinny_kernel,
//   pack_rows_kernel, then the chunked gather in ffn_fused.hip): z goes to an
//   fp32 workspace; the packing kernel takes one workgroup per row, and its
//   last workgroup derives the per-row results (overflow flags and list, work
//   order, tile prefixes and the chunking of the rows' entries).
#include <mutex>

#include "decode.h"
#include "decode2.h"
#include "launch.h"
#include "twell_device.h"
#include "wave_ops.h"

// Workspace of twell_ffn_decode_noalloc, for callers that cannot allocate
// (graph capture, serving loops).  A device array of the code object: every
// GPU the library runs on holds its own copy, at its own address, until the
// process ends.  On the host the array's name is only a stand-in, never a
// device address: host code uses the address hipGetSymbolAddress returns for
// the current device (decode_static_workspace), kept per device.  Calls on
// one GPU share the copy, so calls that overlap in time on one GPU race.
static __device__ __align__(256) char scratch[twell::DEC_STATIC_BYTES];

namespace twell {

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[SCRATCH_MAX_DEVICES];
}  // namespace

hipError_t decode_static_workspace(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

// ------------------------------------------------------------------ gate
// z[m][n0 + n] for the workgroup's 32 neurons n, all rows m < T (MB blocks of
// 32 rows).  The workgroup's 32 rows of W_g (a contiguous d x 64-byte block)
// stream into LDS with global->LDS copies, a stage of up to DEC_KS K elements
// at a time, so the whole stage is in flight at once and no VGPRs hold it;
// the x operands of the wave's K chunks are requested before the copies
// (x is small and shared by all workgroups through L2).  LDS rows hold the
// stage's 16-byte chunks with the chunk index XORed with the row (inside
// groups of 16 chunks; rows padded to a multiple of 256 bytes), so the 16 rows
// one ds_read_b128 phase touches hit 16 distinct bank groups.  K is cut into
// 64-element chunks dealt to the 8 waves round-robin; in a chunk, lane half h
// supplies elements [32 h, 32 h + 32) of its row as four 8-element MFMA
// operands (A and B in the same element order).  The 8 partial 32 x 32 blocks
// are added in LDS in wave order (deterministic).  Block 0 also clears the
// packing kernel's completion counter.
constexpr int DEC_KS = 2048;  // K elements per LDS stage (32 rows x 4 KiB)

__device__ __forceinline__ int skinny_slot(int ch, int n) { return (ch & ~15) | ((ch ^ n) & 15); }

constexpr int DEC_SB = 32 * DEC_KS * 2;  // bytes of the gate's LDS stage buffer

// The skinny gate of one workgroup (512 threads): z[m][n0 + c] for its 32
// neurons c and all rows m < T, written to global memory and, when zs is
// given, to LDS as zs[m * 32 + c].  sb: the DEC_SB-byte stage buffer (free
// again on return).
template <int MB>
__device__ __forceinline__ void skinny_gate(const __bf16 *x, const __bf16 *wg_t, int T, int d, int F, float *z,
                                            char *sb, float *zs)
{
    constexpr int NW = 8, KCW = DEC_KS / 64 / NW;  // K chunks per wave per stage
    static_assert(MB * NW * 16 * 64 * 4 <= DEC_SB, "reduction fits the stage buffer");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 32;
    const int n = lane & 31, h = lane >> 5;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wg_t + (int64_t)n0 * d, (uint32_t)(32 * d * 2));
    const char *arow[MB];
    bool aok[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 32 + n;
        aok[mb] = m < T;
        arow[mb] = reinterpret_cast<const char *>(x + (int64_t)(aok[mb] ? m : 0) * d);
    }
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[mb][i] = 0.f;
    for (int k0 = 0; k0 < d; k0 += DEC_KS) {
        const int ks = d - k0 < DEC_KS ? d - k0 : DEC_KS;  // multiple of 64
        const int cpr = ks / 8;                              // 16-byte chunks per row
        const int spr = (cpr + 15) & ~15;                    // LDS slots per row
        const int nkc = ks / 64;
        // this wave's x operands for the stage
        u32x4 a[KCW][MB][4];
#pragma unroll
        for (int u = 0; u < KCW; ++u) {
            const int kc = wave + u * NW;
            const int off = (k0 + kc * 64 + 32 * h) * 2;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[u][mb][q] = (kc < nkc && aok[mb]) ? ldg16(arow[mb] + off + 16 * q) : u32x4{0, 0, 0, 0};
        }
        // the stage of W_g: 64 slots (1 KiB) per wave instruction
        for (int s0 = wave * 64; s0 < 32 * spr; s0 += NW * 64) {
            const int slot = s0 + lane;
            const int r = slot / spr, sl = slot - r * spr;
            const int ch = skinny_slot(sl, r);
            const int voff = (r * d + k0) * 2 + (ch < cpr ? ch : 0) * 16;  // padding slots re-read chunk 0
            dma16(rw, sb + s0 * 16, voff, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // copies and x loads complete
        wg_barrier();
#pragma unroll
        for (int u = 0; u < KCW; ++u) {
            const int kc = wave + u * NW;
            if (kc < nkc) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ch = kc * 8 + 4 * h + q;
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(sb + (n * spr + skinny_slot(ch, n)) * 16);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        mfma_chunk(__bf16{}, a[u][mb][q], b, acc[mb]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
        wg_barrier();                        // before the next stage (or the reduction) overwrites sb
    }
    float *red = reinterpret_cast<float *>(sb);  // [wave][block][register][lane]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            red[((wave * MB + mb) * 16 + i) * 64 + lane] = acc[mb][i];
    __syncthreads();
    // element (row r, column c) of block mb sits in register i of lane l
    for (int e = tid; e < MB * 1024; e += 512) {
        const int mb = e >> 10, r = (e >> 5) & 31, c = e & 31;
        const int m = mb * 32 + r;
        if (m >= T)
            continue;
        const int l = c + 32 * ((r >> 2) & 1), i = ((r >> 3) << 2) + (r & 3);
        float s = red[((0 * MB + mb) * 16 + i) * 64 + l];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            s += red[((w * MB + mb) * 16 + i) * 64 + l];
        z[(int64_t)m * F + n0 + c] = s;
        if (zs)
            zs[m * 32 + c] = s;
    }
    __syncthreads();  // red (sb) read in full; zs complete
}

template <int MB>
__global__ __launch_bounds__(512) void gate_skinny_kernel(const __bf16 *x, const __bf16 *wg_t, int T, int d,
                                                          int F, float *z, int32_t *counter)
{
    __shared__ __attribute__((aligned(16))) char sb[DEC_SB];
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *counter = 0;
    skinny_gate<MB>(x, wg_t, T, d, F, z, sb, nullptr);
}

// ------------------------------------------------------------------ packing
// One workgroup of 8 waves per row t; wave w packs tiles w, w + 8, ... (the
// z values of up to 4 tiles are requested together).  Per tile, lane l holds
// columns l + 64 j; one ballot per j gives the activity (z > 0) and each
// active column's slot (earlier j's counts plus the active lanes below it):
// ascending columns.  Values are rounded to bf16 (nearest even); slots past
// min(count, cap) are zero.  The row's total and overflow flag are summed in
// LDS.  The workgroup that finishes last (completion counter, device-scope
// fences) then derives every per-row result, one lane per row.
struct PackArgs {
    const float *z;
    int T, F, tile_w, cap, n_b;
    __bf16 *val;
    uint8_t *idx;
    int32_t *cnt;
    int32_t *row_ovf, *ovf_rows, *n_ovf, *order;
    int max_ovf;
    int32_t *counter, *row_e, *row_o, *chunk0, *chunk_e;
};

// Entries per gather chunk: the smallest DEC_MIN_E * 2^m with total <=
// DEC_BASE_CHUNKS chunks of that size (at most DEC_MAX_E).
__device__ __forceinline__ int chunk_entries(int total)
{
    int e = DEC_MIN_E;
    while (e < DEC_MAX_E && (int64_t)e * DEC_BASE_CHUNKS < total)
        e <<= 1;
    return e;
}

// Work class of a row with e stored entries (0: heaviest), as in the batch
// path's order: e >= 256, 192..255, 128..191, 64..127, 32..63, 16..31, 1..15, 0.
__device__ __forceinline__ int work_class_of(int e)
{
    return e >= 256 ? 0 : e >= 192 ? 1 : e >= 128 ? 2 : e >= 64 ? 3 : e >= 32 ? 4 : e >= 16 ? 5 : e >= 1 ? 6 : 7;
}

// Pack tile b of row t (all lanes of the wave); returns its true count.
__device__ __forceinline__ int pack_tile(const PackArgs &a, int t, int b, const float (&v)[4], int lane)
{
    const int w = a.tile_w, cap = a.cap;
    uint64_t bal[4];
    int total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bal[j] = __ballot(lane + 64 * j < w && v[j] > 0.f);
        total += __popcll(bal[j]);
    }
    const int64_t slot0 = ((int64_t)t * a.n_b + b) * cap;
    int base = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
        if (((bal[j] >> lane) & 1ull) && slot < cap) {
            store_elem(a.val + slot0 + slot, v[j]);
            a.idx[slot0 + slot] = (uint8_t)(lane + 64 * j);
        }
        base += __popcll(bal[j]);
    }
    const int kept = total < cap ? total : cap;
    for (int s = kept + lane; s < cap; s += 64) {
        store_elem(a.val + slot0 + s, 0.f);
        a.idx[slot0 + s] = 0;
    }
    if (lane == 0)
        a.cnt[(int64_t)t * a.n_b + b] = total;
    return total;
}

__global__ __launch_bounds__(512) void pack_rows_kernel(PackArgs a)
{
    constexpr int NW = 8, BATCH = 4;
    __shared__ int s_last, s_e[NW], s_o[NW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = blockIdx.x;
    const int w = a.tile_w;
    const float *zr = a.z + (int64_t)t * a.F;
    int e = 0, o = 0;
    for (int b0 = wave; b0 < a.n_b; b0 += NW * BATCH) {
        float v[BATCH][4];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int b = b0 + u * NW;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = lane + 64 * j;
                v[u][j] = (b < a.n_b && c < w) ? zr[(int64_t)b * w + c] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int b = b0 + u * NW;
            if (b < a.n_b) {
                const int tot = pack_tile(a, t, b, v[u], lane);
                e += tot;
                o |= tot > a.cap;
            }
        }
    }
    if (lane == 0) {
        s_e[wave] = e;
        s_o[wave] = o;
    }
    __syncthreads();
    if (tid == 0) {
        int se = 0, so = 0;
        for (int k = 0; k < NW; ++k) {
            se += s_e[k];
            so |= s_o[k];
        }
        a.row_e[t] = se;
        a.row_o[t] = so;
        if (gridDim.x == 1) {
            s_last = 1;  // a single row: this workgroup is the last, no fences needed
        } else {
            __threadfence();
            s_last = atomicAdd(a.counter, 1) == (int)gridDim.x - 1;
        }
    }
    __syncthreads();
    if (!s_last)
        return;
    if (gridDim.x > 1)
        __threadfence();
    if (wave != 0)
        return;
    // one lane per row (T <= 64)
    const bool live = lane < a.T;
    const int re = live ? a.row_e[lane] : 0;
    const int ovf = live ? (a.row_o[lane] != 0) : 0;
    if (live)
        a.row_ovf[lane] = ovf;
    int sum_e;
    (void)wave_excl_scan(re, lane, sum_e);
    const int E = chunk_entries(sum_e);
    const int nch = (re + E - 1) / E;
    int n_chunks;
    const int c0 = wave_excl_scan(nch, lane, n_chunks);
    if (live)
        a.chunk0[lane] = c0;
    if (lane == 0) {
        a.chunk0[a.T] = n_chunks;
        *a.chunk_e = E;
    }
    // ascending overflow list (first max_ovf rows) and its true length
    const uint64_t om = __ballot(live && ovf);
    const int opos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(om >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)om, 0u));
    if (live && ovf && opos < a.max_ovf)
        a.ovf_rows[opos] = lane;
    if (lane == 0)
        *a.n_ovf = __popcll(om);
    // work order: classes of stored entries (0 for overflow rows), heaviest first
    const int cls = work_class_of(ovf ? 0 : re);
    int base = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint64_t m = __ballot(live && cls == k);
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (live && cls == k)
            a.order[pos] = lane;
        base += __popcll(m);
    }
}

// ------------------------------------------------------------------ gate + gather
// The decode step in two kernels.  An entry's contribution to y is
// bf16(z) * (x . W_u^T[j]) * W_d[j] whether or not its row overflows (a row
// that fits keeps every active column in TwELL; an overflow row's entries are
// its dense backup row, the same rounded values), so each gate workgroup can
// do the up/down work of its own 32 neurons as soon as their z is known,
// with nothing from the packing.
//
// gate_gather_kernel: the skinny gate (z to global and LDS), then, for each
// row t, the workgroup's active neurons j (ascending) give the partial row
// P[t][g] = sum_j bf16(z[t][j]) (x[t] . W_u^T[j]) W_d[j] (g = the workgroup),
// written with flag[t][g] = 1 when there is at least one active j (else
// flag = 0 and nothing is written).  Rows are dealt to the 8 waves; with at
// most 4 rows, S waves share a row (S the largest power of two with
// S * T <= 8), wave `sub` taking the entries of rank sub, sub + S, ..., and
// their partial rows are added in LDS in sub order.  A wave streams its entries in
// order with the next entry's W_u^T and W_d rows (and the next row's x)
// requested before the current entry is reduced; each dot product is summed
// over the lane's chunks, then across the wave (DPP, fixed order).
struct GatherArgs {
    const __bf16 *x, *wg_t, *wu_t, *wd;
    int T, d, F;
    float *z;         // [T][F]
    int32_t *flag;    // [T][G]
    float *part;      // [T][G][d]
    int32_t *counter; // cleared here for reduce_pack_kernel
};

template <int NC> struct GEnt {
    u32x4 wu[NC], wd[NC];
};

template <int MB, int NC>
__global__ __launch_bounds__(512) void gate_gather_kernel(GatherArgs a)
{
    __shared__ __attribute__((aligned(16))) char sb[DEC_SB];
    __shared__ float zs[DEC_MAX_T * 32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x, G = gridDim.x, n0 = g * 32;
    const int T = a.T, d = a.d;
    if (g == 0 && tid == 0)
        *a.counter = 0;
    skinny_gate<MB>(a.x, a.wg_t, T, d, a.F, a.z, sb, zs);

    // flags: row t has an active neuron in this workgroup
    if (tid < T) {
        int any = 0;
        for (int c = 0; c < 32; ++c)
            any |= zs[tid * 32 + c] > 0.f;
        a.flag[(int64_t)tid * G + g] = any;
    }
    // waves per row: the largest power of two with S * T <= 8 (so that with
    // S > 1 every wave serves exactly one row and its combine slot)
    const int S = T >= 5 ? 1 : T >= 3 ? 2 : T == 2 ? 4 : 8;
    const int R = 8 / S;                                      // rows dealt at a time
    const int sub = wave % S, rg = wave / S;
    const int nchunks = d / 8;  // 16-byte chunks of a bf16 row
    const int64_t row_bytes = (int64_t)d * 2;
    float *comb = reinterpret_cast<float *>(sb);  // S > 1: [wave][d] partial rows

    // the wave's rows t = rg, rg + R, ... and, per row, its entries: active
    // columns c of rank sub, sub + S, ... (ascending)
    auto row_mask = [&](int t) -> uint32_t {
        const uint64_t b = __ballot(lane < 32 && zs[t * 32 + (lane & 31)] > 0.f);
        uint32_t m = (uint32_t)b;
        if (S > 1) {
            uint32_t keep = 0;
            int rank = 0;
            while (m) {
                const int c = __builtin_ctz(m);
                m &= m - 1;
                if (rank % S == sub)
                    keep |= 1u << c;
                ++rank;
            }
            m = keep;
        }
        return m;
    };
    // cursor: row t (or >= T when done) and its remaining mask
    int t = rg;
    uint32_t m = t < T ? row_mask(t) : 0u;
    auto advance_row = [&]() {
        while (t < T && m == 0u) {
            t += R;
            m = t < T ? row_mask(t) : 0u;
        }
    };
    float yacc[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            yacc[c][e] = 0.f;
    auto load_ent = [&](int c, auto &en) {
        const int64_t j = n0 + c;
        const char *pu = (const char *)a.wu_t + j * row_bytes;
        const char *pd = (const char *)a.wd + j * row_bytes;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int ch = lane + 64 * k;
            const bool ok = ch < nchunks;
            en.wu[k] = ok ? ldg16(pu + ch * 16) : u32x4{0, 0, 0, 0};
            en.wd[k] = ok ? ldg16(pd + ch * 16) : u32x4{0, 0, 0, 0};
        }
    };
    auto load_x = [&](int tt, u32x4 (&xv)[NC]) {
        const char *px = (const char *)a.x + (int64_t)tt * row_bytes;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int ch = lane + 64 * k;
            xv[k] = ch < nchunks ? ldg16(px + ch * 16) : u32x4{0, 0, 0, 0};
        }
    };
    auto write_row = [&](int tt) {
        float *pr = a.part + ((int64_t)tt * G + g) * d;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int ch = lane + 64 * k;
            if (ch < nchunks) {
                *reinterpret_cast<float4 *>(pr + ch * 8) = make_float4(yacc[k][0], yacc[k][1], yacc[k][2], yacc[k][3]);
                *reinterpret_cast<float4 *>(pr + ch * 8 + 4) =
                    make_float4(yacc[k][4], yacc[k][5], yacc[k][6], yacc[k][7]);
            }
        }
    };
    auto write_comb = [&]() {
        float *pr = comb + (int64_t)wave * d;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int ch = lane + 64 * k;
            if (ch < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pr[ch * 8 + e] = yacc[k][e];
            }
        }
    };

    // PF: the next entry's rows are requested before this one is reduced (a
    // second set of row registers; at d = 4096 that would spill, so there
    // the entries go one after another)
    constexpr bool PF = NC <= 4;
    advance_row();
    if (t < T) {
        u32x4 xa[NC], xb[PF ? NC : 1];
        GEnt<NC> ea;
        GEnt<PF ? NC : 1> eb;
        int ct = t, cc = __builtin_ctz(m);
        m &= m - 1;
        load_x(ct, xa);
        load_ent(cc, ea);
        while (true) {
            // the next entry: the rest of this row, else the next row with entries
            advance_row();
            const bool more = t < T;
            int nt = t, nc = 0;
            if (more) {
                nc = __builtin_ctz(m);
                m &= m - 1;
                if constexpr (PF) {
                    load_ent(nc, eb);
                    if (nt != ct)
                        load_x(nt, xb);
                }
            }
            // this entry: u = x[ct] . W_u^T[j], then y += bf16(z) u W_d[j]
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    part = fmaf(chunk_elem<__bf16>(xa[k], e), chunk_elem<__bf16>(ea.wu[k], e), part);
            const float u = wave_sum(part);
            const float hv = (float)(__bf16)zs[ct * 32 + cc];
            const float sc = hv * u;
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    yacc[k][e] = fmaf(sc, chunk_elem<__bf16>(ea.wd[k], e), yacc[k][e]);
            if (!more || nt != ct) {
                // the row is done
                if (S == 1)
                    write_row(ct);
                else
                    write_comb();
#pragma unroll
                for (int k = 0; k < NC; ++k)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        yacc[k][e] = 0.f;
                if constexpr (PF) {
                    if (more)
#pragma unroll
                        for (int k = 0; k < NC; ++k)
                            xa[k] = xb[k];
                }
            }
            if (!more)
                break;
            if constexpr (PF) {
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    ea.wu[k] = eb.wu[k];
                    ea.wd[k] = eb.wd[k];
                }
            } else {
                load_ent(nc, ea);
                if (nt != ct)
                    load_x(nt, xa);
            }
            ct = nt;
            cc = nc;
        }
    } else if (S > 1) {
        write_comb();  // zeros: this wave had no entries
    }
    if (S > 1) {
        // S > 1: T <= 4 rows, wave w = t * S + sub holds a part of row t's
        // partial row (zeros when it had no entries); add them in sub order
        // (waves of rows past T took no entries and are not read)
        __syncthreads();
        for (int tt = 0; tt < T; ++tt) {
            bool any = false;  // the same in every thread (flag 0: nothing to write)
            for (int c = 0; c < 32; ++c)
                any |= zs[tt * 32 + c] > 0.f;
            if (!any)
                continue;
            float *pr = a.part + ((int64_t)tt * G + g) * d;
            for (int col = tid; col < d; col += 512) {
                float v = comb[(int64_t)(tt * S) * d + col];
                for (int q = 1; q < S; ++q)
                    v += comb[(int64_t)(tt * S + q) * d + col];
                pr[col] = v;
            }
        }
    }
}

// reduce_pack_kernel, after gate_gather_kernel: blocks [0, T * CB) add row
// t's partial rows in workgroup order into y[t] (CB blocks of 1024 columns
// per row, 4 columns per thread; the flagged workgroups are listed in LDS
// first, so the adds run in a fixed order with several loads in flight);
// blocks [T * CB, T * CB + n_b) pack TwELL tile b of every row from z (the
// batch epilogue's rules); the packing block that finishes last (completion
// counter cleared by gate_gather_kernel, device-scope fences, no waiting)
// writes the per-row results: overflow flags, the ascending overflow list and
// its count, the work order, and the dense backup rows ReLU(z) (bf16) of the
// first min(n_ovf, max_ovf) overflow rows.
struct ReducePackArgs {
    PackArgs pk;        // z, T, F, tile_w, cap, n_b, val, idx, cnt, row_ovf, ovf_rows, n_ovf, order, max_ovf, counter
    const int32_t *flag;
    const float *part;
    float *y;
    int d, G, CB;
    __bf16 *dense;
};

__global__ __launch_bounds__(256) void reduce_pack_kernel(ReducePackArgs a)
{
    __shared__ int slist[DEC_MAX_G];
    __shared__ int scount[4];
    __shared__ int s_last;
    __shared__ int s_ovf[DEC_MAX_T], s_re[DEC_MAX_T], s_ov[DEC_MAX_T];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const PackArgs &pk = a.pk;
    const int T = pk.T, G = a.G, d = a.d;
    const int nred = T * a.CB;
    if ((int)blockIdx.x < nred) {
        const int t = blockIdx.x / a.CB, cb = blockIdx.x - t * a.CB;
        // ascending list of the flagged workgroups of row t
        int n = 0;
        for (int g0 = 0; g0 < G; g0 += 256) {
            const int gg = g0 + tid;
            const bool f = gg < G && a.flag[(int64_t)t * G + gg] != 0;
            const uint64_t b = __ballot(f);
            const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (lane == 0)
                scount[wave] = __popcll(b);
            __syncthreads();
            int base = n;
            for (int w = 0; w < wave; ++w)
                base += scount[w];
            if (f)
                slist[base + below] = gg;
            n += scount[0] + scount[1] + scount[2] + scount[3];
            __syncthreads();
        }
        const int col = cb * 1024 + tid * 4;
        if (col < d) {
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
            const float *pr = a.part + (int64_t)t * G * d + col;
            // 32 partial rows requested at a time, added in list order
            constexpr int B = 32;
            for (int k = 0; k < n; k += B) {
                float4 v[B];
#pragma unroll
                for (int q = 0; q < B; ++q)
                    v[q] = k + q < n ? *reinterpret_cast<const float4 *>(pr + (int64_t)slist[k + q] * d)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int q = 0; q < B; ++q) {
                    if (k + q < n) {
                        s.x += v[q].x;
                        s.y += v[q].y;
                        s.z += v[q].z;
                        s.w += v[q].w;
                    }
                }
            }
            *reinterpret_cast<float4 *>(a.y + (int64_t)t * d + col) = s;
        }
        return;
    }
    // packing of tile b, rows t = wave, wave + 4, ... (at most 16 per wave):
    // every z value of the wave's rows is requested first, so the packing
    // waits for one round of loads, not one per row
    const int b = blockIdx.x - nred;
    const int w = pk.tile_w;
    constexpr int RPW = DEC_MAX_T / 4;
    float v[RPW][4];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int t = wave + 4 * k;
        const float *zr = pk.z + (int64_t)t * pk.F + (int64_t)b * w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = lane + 64 * j;
            v[k][j] = (t < T && c < w) ? zr[c] : 0.f;
        }
    }
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int t = wave + 4 * k;
        if (t < T)
            (void)pack_tile(pk, t, b, v[k], lane);
    }
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        s_last = atomicAdd(pk.counter, 1) == pk.n_b - 1;
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    {
        // stored entries and overflow flag of each row from its tile counts:
        // 4 threads per row (T <= 64), 8 loads in flight each, combined in
        // the lanes' fixed order
        const int t = tid >> 2, qq = tid & 3;
        int re = 0, ov = 0;
        if (t < T) {
            const int32_t *cr = pk.cnt + (int64_t)t * pk.n_b;
            for (int b0 = qq; b0 < pk.n_b; b0 += 32) {
                int cv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    cv[u] = b0 + 4 * u < pk.n_b ? cr[b0 + 4 * u] : 0;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    re += cv[u] < pk.cap ? cv[u] : pk.cap;
                    ov |= cv[u] > pk.cap;
                }
            }
        }
        re += __shfl_xor(re, 1, 64);
        re += __shfl_xor(re, 2, 64);
        ov |= __shfl_xor(ov, 1, 64);
        ov |= __shfl_xor(ov, 2, 64);
        if (qq == 0 && t < T) {
            s_re[t] = re;
            s_ov[t] = ov;
        }
    }
    __syncthreads();
    if (wave == 0) {
        // one lane per row
        const bool live = lane < T;
        const int re = live ? s_re[lane] : 0;
        const int ovf = live ? s_ov[lane] : 0;
        if (live)
            pk.row_ovf[lane] = ovf;
        const uint64_t om = __ballot(live && ovf);
        const int opos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(om >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)om, 0u));
        if (live && ovf && opos < pk.max_ovf) {
            pk.ovf_rows[opos] = lane;
            s_ovf[opos] = lane;
        }
        if (lane == 0) {
            *pk.n_ovf = __popcll(om);
            scount[0] = __popcll(om) < pk.max_ovf ? __popcll(om) : pk.max_ovf;
        }
        // work order: classes of stored entries (0 for overflow rows), heaviest first
        const int cls = work_class_of(ovf ? 0 : re);
        int base = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint64_t mk = __ballot(live && cls == k);
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
            if (live && cls == k)
                pk.order[pos] = lane;
            base += __popcll(mk);
        }
    }
    __syncthreads();
    // dense backup rows of the first min(n_ovf, max_ovf) overflow rows
    const int nv = scount[0];
    for (int i = 0; i < nv; ++i) {
        const float *zr = pk.z + (int64_t)s_ovf[i] * pk.F;
        __bf16 *dr = a.dense + (int64_t)i * pk.F;
#pragma unroll 4
        for (int j = tid * 8; j < pk.F; j += 256 * 8) {
            const float4 p = *reinterpret_cast<const float4 *>(zr + j);
            const float4 q = *reinterpret_cast<const float4 *>(zr + j + 4);
            const float vv[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
            uint32_t hh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                hh[e] = __builtin_bit_cast(uint16_t, (__bf16)(vv[e] > 0.f ? vv[e] : 0.f));
            *reinterpret_cast<u32x4 *>(dr + j) =
                u32x4{hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16), hh[4] | (hh[5] << 16), hh[6] | (hh[7] << 16)};
        }
    }
}

// ------------------------------------------------------------------ launchers
DecodeWs decode_ws_layout(void *base, int T, int F, int tile_w, int d)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    (void)tile_w;
    const size_t o_z = 0;
    const size_t o_ctr = o_z + up((size_t)T * F * 4);
    const size_t o_rows = o_ctr + 256;
    const size_t o_c0 = o_rows + up((size_t)T * 8);
    const size_t o_part = o_c0 + up((size_t)(T + 1) * 4);
    DecodeWs w{};
    w.max_chunks = DEC_BASE_CHUNKS + T;
    w.bytes = o_part + up((size_t)w.max_chunks * d * 4);
    if (base) {
        char *p = static_cast<char *>(base);
        w.z = reinterpret_cast<float *>(p + o_z);
        w.counter = reinterpret_cast<int32_t *>(p + o_ctr);
        w.chunk_e = w.counter + 1;
        w.row_e = reinterpret_cast<int32_t *>(p + o_rows);
        w.row_o = w.row_e + T;
        w.chunk0 = reinterpret_cast<int32_t *>(p + o_c0);
        w.part = reinterpret_cast<float *>(p + o_part);
    }
    return w;
}

DecodeWs2 decode_ws2_layout(void *base, int T, int F, int d)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const int G = F / 32;
    const size_t o_z = 0;
    const size_t o_ctr = o_z + up((size_t)T * F * 4);
    const size_t o_flag = o_ctr + 256;
    const size_t o_part = o_flag + up((size_t)T * G * 4);
    DecodeWs2 w{};
    w.bytes = o_part + up((size_t)T * G * d * 4);
    if (base) {
        char *p = static_cast<char *>(base);
        w.z = reinterpret_cast<float *>(p + o_z);
        w.counter = reinterpret_cast<int32_t *>(p + o_ctr);
        w.flag = reinterpret_cast<int32_t *>(p + o_flag);
        w.part = reinterpret_cast<float *>(p + o_part);
    }
    return w;
}

template <int MB>
static void gather_go(const GatherArgs &a, int nc, hipStream_t s)
{
    const dim3 grid(a.F / 32), block(512);
    if (nc <= 1)
        gate_gather_kernel<MB, 1><<<grid, block, 0, s>>>(a);
    else if (nc <= 2)
        gate_gather_kernel<MB, 2><<<grid, block, 0, s>>>(a);
    else if (nc <= 4)
        gate_gather_kernel<MB, 4><<<grid, block, 0, s>>>(a);
    else
        gate_gather_kernel<MB, 8><<<grid, block, 0, s>>>(a);
}

hipError_t launch_decode2(const void *x, const void *wg_t, const void *wu_t, const void *wd, int T, int d, int F,
                          int tile_w, int cap, void *val, uint8_t *idx, int32_t *cnt, int32_t *row_ovf,
                          int32_t *ovf_rows, int32_t *n_ovf, int32_t *order, int max_ovf, void *dense, float *y,
                          const DecodeWs2 &w, hipStream_t s)
{
    GatherArgs ga{static_cast<const __bf16 *>(x), static_cast<const __bf16 *>(wg_t), static_cast<const __bf16 *>(wu_t),
                  static_cast<const __bf16 *>(wd), T, d, F, w.z, w.flag, w.part, w.counter};
    const int nc = (d / 8 + 63) / 64;  // 16-byte chunks of a row per lane
    if (T <= 32)
        gather_go<1>(ga, nc, s);
    else
        gather_go<2>(ga, nc, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    ReducePackArgs ra{};
    ra.pk = PackArgs{w.z, T, F, tile_w, cap, F / tile_w, static_cast<__bf16 *>(val), idx, cnt, row_ovf, ovf_rows,
                     n_ovf, order, max_ovf, w.counter, nullptr, nullptr, nullptr, nullptr};
    ra.flag = w.flag;
    ra.part = w.part;
    ra.y = y;
    ra.d = d;
    ra.G = F / 32;
    ra.CB = (d + 1023) / 1024;
    ra.dense = static_cast<__bf16 *>(dense);
    reduce_pack_kernel<<<dim3(T * ra.CB + F / tile_w), dim3(256), 0, s>>>(ra);
    return hipGetLastError();
}

hipError_t launch_decode_gate_pack(const void *x, const void *wg_t, int T, int d, int F, int tile_w, int cap,
                                   void *val, uint8_t *idx, int32_t *cnt, int32_t *row_ovf, int32_t *ovf_rows,
                                   int32_t *n_ovf, int32_t *order, int max_ovf, const DecodeWs &w, hipStream_t s)
{
    const __bf16 *xb = static_cast<const __bf16 *>(x);
    const __bf16 *wb = static_cast<const __bf16 *>(wg_t);
    if (T <= 32)
        gate_skinny_kernel<1><<<dim3(F / 32), dim3(512), 0, s>>>(xb, wb, T, d, F, w.z, w.counter);
    else
        gate_skinny_kernel<2><<<dim3(F / 32), dim3(512), 0, s>>>(xb, wb, T, d, F, w.z, w.counter);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    PackArgs a{w.z, T, F, tile_w, cap, F / tile_w, static_cast<__bf16 *>(val), idx, cnt,
               row_ovf, ovf_rows, n_ovf, order, max_ovf, w.counter, w.row_e, w.row_o, w.chunk0, w.chunk_e};
    pack_rows_kernel<<<dim3(T), dim3(512), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace twell
