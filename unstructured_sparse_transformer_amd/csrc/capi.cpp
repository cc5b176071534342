// capi.cpp -- the C ABI declared in include/twell.h: argument checks on the
// host, then launches on the caller's stream.  Nothing here allocates or
// synchronises; the only state kept between calls is the per-device address
// of twell_ffn_decode_noalloc's static scratch (decode.hip).
#include "twell.h"

#include <hip/hip_runtime.h>

#include "decode2.h"
#include "launch.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t vdtype) { return vdtype == TWELL_BF16 ? 2 : 4; }

// Shape / type rules shared by every call.
int check_layout(const twell_t *h, int32_t d)
{
    if (!h)
        return TWELL_E_NULL;
    if (h->vdtype != TWELL_F32 && h->vdtype != TWELL_BF16)
        return TWELL_E_UNSUPPORTED;
    const int w = h->tile_w;
    if (w != 32 && w != 64 && w != 128 && w != 256)
        return TWELL_E_UNSUPPORTED;
    if (h->cap < 1 || h->cap > w)
        return TWELL_E_UNSUPPORTED;
    if (h->T < 0 || h->F <= 0 || h->F % w != 0 || h->F % 64 != 0 || d <= 0 || d % 64 != 0)
        return TWELL_E_SHAPE;
    // The fused step keeps a token's row in registers: at most 8 KiB per row.
    if ((int64_t)d * elem_size(h->vdtype) > 8192)
        return TWELL_E_UNSUPPORTED;
    // GEMM operands are addressed with 32-bit byte offsets: each matrix < 4 GiB;
    // TwELL slots with 32-bit element offsets: T * n_b * cap < 2^31.
    const int64_t lim = (int64_t)1 << 32;
    if ((int64_t)h->T * d * elem_size(h->vdtype) >= lim || (int64_t)h->F * d * elem_size(h->vdtype) >= lim)
        return TWELL_E_SHAPE;
    if ((int64_t)h->T * (h->F / w) * h->cap >= ((int64_t)1 << 31))
        return TWELL_E_SHAPE;
    return TWELL_OK;
}

int check_ptrs(const twell_t *h)
{
    if (!h->val || !h->idx || !h->cnt)
        return TWELL_E_NULL;
    // val / idx / cnt are addressed element-wise; natural alignment suffices.
    if ((reinterpret_cast<uintptr_t>(h->val) & (elem_size(h->vdtype) - 1)) != 0 ||
        (reinterpret_cast<uintptr_t>(h->cnt) & 3u) != 0)
        return TWELL_E_ALIGN;
    return TWELL_OK;
}

int check_mat(const void *p)
{
    if (!p)
        return TWELL_E_NULL;
    return aligned16(p) ? TWELL_OK : TWELL_E_ALIGN;
}

int check_hybrid(const twell_hybrid_t *hy)
{
    if (!hy)
        return TWELL_E_NULL;
    if (hy->max_ovf < 0 || (int64_t)hy->max_ovf * hy->ell.F * elem_size(hy->ell.vdtype) >= ((int64_t)1 << 32))
        return TWELL_E_SHAPE;
    if (hy->ell.T == 0)
        return TWELL_OK;
    if (!hy->row_ovf || !hy->n_ovf || !hy->order)
        return TWELL_E_NULL;
    if (hy->max_ovf > 0 && (!hy->ovf_rows || !hy->dense))
        return TWELL_E_NULL;
    if (hy->max_ovf > 0 && !aligned16(hy->dense))
        return TWELL_E_ALIGN;
    if ((reinterpret_cast<uintptr_t>(hy->row_ovf) & 3u) || (reinterpret_cast<uintptr_t>(hy->ovf_rows) & 3u) ||
        (reinterpret_cast<uintptr_t>(hy->n_ovf) & 3u) || (reinterpret_cast<uintptr_t>(hy->order) & 3u))
        return TWELL_E_ALIGN;
    return TWELL_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TWELL_OK : TWELL_E_HIP; }

#define TWELL_TRY(expr)                  \
    do {                                 \
        const int _st = (expr);          \
        if (_st != TWELL_OK)             \
            return _st;                  \
    } while (0)

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the calls that take one (the fused step and the overflow FFN),
// 256-byte aligned sections: the fused step's (twell::fused_ws_layout: packed
// entries, entry counts, partial dot products), the overflow rows' gated
// products [max_ovf][F] (vdtype), and the down projection's split-K partial
// slabs [splits][max_ovf][d] fp32.
struct Ws {
    size_t s_off, p_off, part_off, bytes;
    int splits;
};

Ws ws_layout(int32_t T, int32_t F, int32_t tile_w, int32_t cap, int32_t max_ovf, int32_t d, int32_t vdtype)
{
    Ws w{};
    w.s_off = 0;
    w.p_off = up256(twell::fused_ws_layout(nullptr, T, F, tile_w, cap, d, elem_size(vdtype)).bytes);
    w.splits = max_ovf > 0 ? twell::down_splits(max_ovf, F, d) : 1;
    w.part_off = w.p_off + (max_ovf > 0 ? up256((size_t)max_ovf * (size_t)F * (size_t)elem_size(vdtype)) : 0);
    w.bytes = w.part_off + (max_ovf > 0 && w.splits > 1 ? (size_t)w.splits * max_ovf * d * sizeof(float) : 0);
    return w;
}

Ws ws_layout(const twell_hybrid_t *hy, int32_t d)
{
    const twell_t *h = &hy->ell;
    return ws_layout(h->T, h->F, h->tile_w, h->cap, hy->max_ovf, d, h->vdtype);
}

// The workspace argument against a layout's size.
int check_ws(const void *workspace, size_t workspace_bytes, size_t need)
{
    if (need == 0)
        return TWELL_OK;
    if (!workspace || workspace_bytes < need)
        return TWELL_E_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return TWELL_E_ALIGN;
    return TWELL_OK;
}

// Checks shared by twell_ffn_from_gate and twell_ffn_forward (T > 0).
int check_layer(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                const twell_hybrid_t *hy, const float *y, const void *workspace, size_t workspace_bytes)
{
    const twell_t *h = &hy->ell;
    TWELL_TRY(check_ptrs(h));
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wg_t));
    TWELL_TRY(check_mat(wu_t));
    TWELL_TRY(check_mat(wd));
    TWELL_TRY(check_mat(y));
    return check_ws(workspace, workspace_bytes, ws_layout(hy, d).bytes);
}

// The layer after the gate, arguments already checked: the fused step's
// entries kernel (which also writes the overflow flags and work values), the
// overflow list and work order, the fused step's two passes, then the dense
// backup and gated up product of the overflow rows in one GEMM, and their
// down projection.
int launch_from_gate(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                     const twell_hybrid_t *hy, float *y, void *workspace, hipStream_t s)
{
    const twell_t *h = &hy->ell;
    const Ws w = ws_layout(hy, d);
    char *ws = static_cast<char *>(workspace);
    TWELL_TRY(hip_status(twell::launch_ffn_entries(h->vdtype, h->cnt, h->val, h->idx, h->T, h->F, h->tile_w, h->cap,
                                                   d, ws + w.s_off, hy->row_ovf, hy->order, s)));
    const twell::FusedWs fw = twell::fused_ws_layout(ws + w.s_off, h->T, h->F, h->tile_w, h->cap, d,
                                                     elem_size(h->vdtype));
    TWELL_TRY(hip_status(twell::launch_compact_rows(hy->row_ovf, h->T, hy->max_ovf, hy->ovf_rows, hy->n_ovf,
                                                    hy->order, s, fw.order_e)));
    TWELL_TRY(hip_status(twell::launch_ffn_passes(h->vdtype, h->cnt, h->val, h->idx, hy->order, h->T, h->F,
                                                  h->tile_w, h->cap, x, wu_t, wd, d, y, ws + w.s_off, true, s)));
    if (hy->max_ovf == 0)
        return TWELL_OK;
    void *pbuf = ws + w.p_off;
    float *part = w.splits > 1 ? reinterpret_cast<float *>(ws + w.part_off) : nullptr;
    TWELL_TRY(hip_status(twell::launch_dense_gate_up(h->vdtype, x, h->T, wg_t, wu_t, hy->ovf_rows, hy->n_ovf,
                                                     hy->max_ovf, d, h->F, hy->dense, pbuf, s)));
    return hip_status(twell::launch_down(h->vdtype, pbuf, wd, hy->ovf_rows, hy->n_ovf, hy->max_ovf, h->F, d, y, part,
                                         w.splits, s));
}

// Checks of the decode-shaped calls, apart from their workspace (T == 0
// passes once the shape is valid).
int check_decode(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                 const twell_hybrid_t *hy, const float *y)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *h = &hy->ell;
    TWELL_TRY(check_layout(h, d));
    TWELL_TRY(check_hybrid(hy));
    if (h->vdtype != TWELL_BF16 || h->T > twell::DEC_MAX_T || (int64_t)h->T * h->F > twell::DEC_MAX_TF ||
        h->F / h->tile_w > twell::DEC_MAX_NB)
        return TWELL_E_UNSUPPORTED;
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wg_t));
    TWELL_TRY(check_mat(wu_t));
    TWELL_TRY(check_mat(wd));
    TWELL_TRY(check_mat(y));
    return check_ptrs(h);
}

// The decode-shaped layer on a carved workspace, arguments already checked.
int launch_decode(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                  const twell_hybrid_t *hy, float *y, const twell::DecodeWs &w, hipStream_t s)
{
    const twell_t *h = &hy->ell;
    TWELL_TRY(hip_status(twell::launch_decode_gate_pack(x, wg_t, h->T, d, h->F, h->tile_w, h->cap, h->val, h->idx,
                                                        h->cnt, hy->row_ovf, hy->ovf_rows, hy->n_ovf, hy->order,
                                                        hy->max_ovf, w, s)));
    return hip_status(twell::launch_ffn_decode(h->cnt, h->val, h->idx, h->T, h->F, h->tile_w, h->cap, x, wu_t, wd, d,
                                               hy->row_ovf, hy->ovf_rows, hy->n_ovf, hy->max_ovf, hy->dense, y, w, s));
}

}  // namespace

extern "C" {

int twell_version(void) { return 201; }

const char *twell_status_str(int status)
{
    switch (status) {
    case TWELL_OK:
        return "ok";
    case TWELL_E_NULL:
        return "a required pointer is NULL";
    case TWELL_E_ALIGN:
        return "a device pointer is not suitably aligned (16 bytes for x, weights, y, dense)";
    case TWELL_E_SHAPE:
        return "bad shape (need T >= 0, d % 64 == 0, F % tile_w == 0, F % 64 == 0)";
    case TWELL_E_UNSUPPORTED:
        return "unsupported tile width / capacity / dtype / model width";
    case TWELL_E_HIP:
        return "HIP launch failed";
    case TWELL_E_WORKSPACE:
        return "workspace missing or too small";
    case TWELL_E_SCRATCH:
        return "the call needs more scratch than the library's static array holds (16 MiB per GPU)";
    default:
        return "unknown status";
    }
}

int twell_pack_gate(const void *x, const void *wg_t, int32_t d, const twell_t *h, void *stream)
{
    TWELL_TRY(check_layout(h, d));
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wg_t));
    TWELL_TRY(check_ptrs(h));
    return hip_status(twell::launch_gate_twell(h->vdtype, x, wg_t, h->T, d, h->F, h->tile_w, h->cap, h->val, h->idx,
                                               h->cnt, static_cast<hipStream_t>(stream)));
}

int twell_gate_dense(const void *x, const void *wg_t, int32_t d, int32_t T, int32_t F, int32_t vdtype, void *h,
                     void *stream)
{
    if (vdtype != TWELL_F32 && vdtype != TWELL_BF16)
        return TWELL_E_UNSUPPORTED;
    if (T < 0 || F <= 0 || F % 64 != 0 || d <= 0 || d % 64 != 0)
        return TWELL_E_SHAPE;
    const int64_t lim = (int64_t)1 << 32;
    if ((int64_t)T * d * elem_size(vdtype) >= lim || (int64_t)F * d * elem_size(vdtype) >= lim)
        return TWELL_E_SHAPE;
    if (T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wg_t));
    if (!h)
        return TWELL_E_NULL;
    if ((reinterpret_cast<uintptr_t>(h) & (elem_size(vdtype) - 1)) != 0)
        return TWELL_E_ALIGN;
    return hip_status(twell::launch_gate_dense(vdtype, x, wg_t, T, d, F, h, static_cast<hipStream_t>(stream)));
}

int twell_pack_gate_stats(const void *x, const void *wg_t, int32_t d, const twell_t *h, int32_t *neuron_cnt,
                          float *l1, void *stream)
{
    TWELL_TRY(check_layout(h, d));
    if (!neuron_cnt || !l1)
        return TWELL_E_NULL;
    if ((reinterpret_cast<uintptr_t>(neuron_cnt) | reinterpret_cast<uintptr_t>(l1)) & 3u)
        return TWELL_E_ALIGN;
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wg_t));
    TWELL_TRY(check_ptrs(h));
    return hip_status(twell::launch_gate_twell_stats(h->vdtype, x, wg_t, h->T, d, h->F, h->tile_w, h->cap, h->val,
                                                     h->idx, h->cnt, neuron_cnt, l1,
                                                     static_cast<hipStream_t>(stream)));
}

int twell_partition_overflow(const void *x, const void *wg_t, int32_t d, const twell_hybrid_t *hy, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *h = &hy->ell;
    TWELL_TRY(check_layout(h, d));
    TWELL_TRY(check_hybrid(hy));
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wg_t));
    if (!h->cnt)
        return TWELL_E_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n_b = h->F / h->tile_w;
    TWELL_TRY(hip_status(twell::launch_row_flags(h->cnt, h->T, n_b, h->cap, hy->row_ovf, hy->order, s)));
    TWELL_TRY(hip_status(
        twell::launch_compact_rows(hy->row_ovf, h->T, hy->max_ovf, hy->ovf_rows, hy->n_ovf, hy->order, s)));
    return hip_status(twell::launch_dense_gate(h->vdtype, x, h->T, wg_t, hy->ovf_rows, hy->n_ovf, hy->max_ovf, d, h->F,
                                               hy->dense, s));
}

int twell_pack_gate_hybrid(const void *x, const void *wg_t, int32_t d, const twell_hybrid_t *hy, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    TWELL_TRY(check_layout(&hy->ell, d));
    TWELL_TRY(check_hybrid(hy));
    TWELL_TRY(twell_pack_gate(x, wg_t, d, &hy->ell, stream));
    return twell_partition_overflow(x, wg_t, d, hy, stream);
}

int twell_dense_to_hybrid(const void *h, const twell_hybrid_t *hy, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *e = &hy->ell;
    TWELL_TRY(check_layout(e, 64));
    TWELL_TRY(check_hybrid(hy));
    if (e->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(h));
    TWELL_TRY(check_ptrs(e));
    return hip_status(twell::launch_dense_to_hybrid(e->vdtype, h, e->T, e->F, e->tile_w, e->cap, e->val, e->idx,
                                                    e->cnt, hy->row_ovf, hy->ovf_rows, hy->n_ovf, hy->order,
                                                    hy->max_ovf, hy->dense, static_cast<hipStream_t>(stream)));
}

int twell_hybrid_to_dense(const twell_hybrid_t *hy, void *out, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *e = &hy->ell;
    TWELL_TRY(check_layout(e, 64));
    TWELL_TRY(check_hybrid(hy));
    if (e->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(out));
    TWELL_TRY(check_ptrs(e));
    return hip_status(twell::launch_hybrid_to_dense(e->vdtype, e->cnt, e->val, e->idx, e->T, e->F, e->tile_w, e->cap,
                                                    hy->ovf_rows, hy->n_ovf, hy->max_ovf, hy->dense, out,
                                                    static_cast<hipStream_t>(stream)));
}

static_assert(sizeof(twell_compact_header_t) == 80, "compact header layout");

size_t twell_compact_min_bytes(int32_t T)
{
    if (T < 0)
        return 0;
    return 256 + (((size_t)(T + 1) * 4 + 255) & ~(size_t)255);
}

int twell_compact_hybrid(const twell_hybrid_t *hy, void *buf, size_t buf_bytes, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *e = &hy->ell;
    TWELL_TRY(check_layout(e, 64));
    TWELL_TRY(check_hybrid(hy));
    if (e->F > 65536 || e->F / e->tile_w > twell::DEC_MAX_NB)
        return TWELL_E_UNSUPPORTED;
    if (!buf)
        return TWELL_E_NULL;
    if (reinterpret_cast<uintptr_t>(buf) & 255u)
        return TWELL_E_ALIGN;
    if (buf_bytes < twell_compact_min_bytes(e->T))
        return TWELL_E_WORKSPACE;
    if (e->T > 0)
        TWELL_TRY(check_ptrs(e));
    return hip_status(twell::launch_compact_hybrid(e->vdtype, e->cnt, e->val, e->idx, hy->row_ovf, hy->ovf_rows,
                                                   hy->n_ovf, hy->max_ovf, hy->dense, e->T, e->F, e->tile_w, e->cap,
                                                   buf, (int64_t)buf_bytes, static_cast<hipStream_t>(stream)));
}

int twell_compact_to_dense(const void *buf, int32_t T, int32_t F, int32_t vdtype, void *out, void *stream)
{
    if (vdtype != TWELL_F32 && vdtype != TWELL_BF16)
        return TWELL_E_UNSUPPORTED;
    if (T < 0 || F <= 0 || F % 64 != 0)
        return TWELL_E_SHAPE;
    if (T == 0)
        return TWELL_OK;
    if (!buf || !out)
        return TWELL_E_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 255u) || !aligned16(out))
        return TWELL_E_ALIGN;
    return hip_status(twell::launch_compact_to_dense(vdtype, buf, T, F, out, static_cast<hipStream_t>(stream)));
}

size_t twell_ffn_backward_workspace_bytes(int32_t T, int32_t F, int32_t d, int32_t max_entries)
{
    if (T < 0 || F <= 0 || d <= 0 || max_entries < 0)
        return 0;
    return twell::bw_ws_layout(nullptr, T, F, d, max_entries).bytes;
}

int twell_ffn_backward(const twell_hybrid_t *hy, const void *x, const void *wg_t, const void *wu_t, const void *wd,
                       int32_t d, const float *dy, float *dx, float *dwg, float *dwu, float *dwd,
                       int32_t max_entries, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *e = &hy->ell;
    TWELL_TRY(check_layout(e, d));
    TWELL_TRY(check_hybrid(hy));
    if (e->vdtype != TWELL_BF16 || d > twell::BW_MAX_D || e->F / e->tile_w > twell::BW_MAX_NB)
        return TWELL_E_UNSUPPORTED;
    if (max_entries < 0)
        return TWELL_E_SHAPE;
    // The entry scan counts in int32: the stored entries of the rows that fit
    // (at most T * n_b * cap) plus the nonzeros of the held dense rows (at
    // most max_ovf * F) must stay below 2^31.
    if ((int64_t)e->T * (e->F / e->tile_w) * e->cap + (int64_t)hy->max_ovf * e->F >= ((int64_t)1 << 31))
        return TWELL_E_SHAPE;
    TWELL_TRY(check_mat(wg_t));
    TWELL_TRY(check_mat(wu_t));
    TWELL_TRY(check_mat(wd));
    TWELL_TRY(check_mat(dwg));
    TWELL_TRY(check_mat(dwu));
    TWELL_TRY(check_mat(dwd));
    if (!workspace)
        return TWELL_E_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return TWELL_E_ALIGN;
    const twell::BwWs w = twell::bw_ws_layout(workspace, e->T, e->F, d, max_entries);
    if (workspace_bytes < w.bytes)
        return TWELL_E_WORKSPACE;
    if (e->T > 0) {
        TWELL_TRY(check_mat(x));
        TWELL_TRY(check_mat(dy));
        TWELL_TRY(check_mat(dx));
        TWELL_TRY(check_ptrs(e));
    }
    twell::BwArgs a{};
    a.T = e->T;
    a.F = e->F;
    a.tile_w = e->tile_w;
    a.cap = e->cap;
    a.n_b = e->F / e->tile_w;
    a.d = d;
    a.nchunks = d * 2 / 16;
    a.n_rc = (e->T + twell::BW_RC - 1) / twell::BW_RC;
    a.max_entries = max_entries;
    a.max_ovf = hy->max_ovf;
    a.cnt = e->cnt;
    a.val = static_cast<const __bf16 *>(e->val);
    a.idx = e->idx;
    a.row_ovf = hy->row_ovf;
    a.ovf_rows = hy->ovf_rows;
    a.n_ovf = hy->n_ovf;
    a.dense = static_cast<const __bf16 *>(hy->dense);
    a.x = static_cast<const __bf16 *>(x);
    a.wg_t = static_cast<const __bf16 *>(wg_t);
    a.wu_t = static_cast<const __bf16 *>(wu_t);
    a.wd = static_cast<const __bf16 *>(wd);
    a.dy = dy;
    a.dx = dx;
    a.dwg = dwg;
    a.dwu = dwu;
    a.dwd = dwd;
    a.ws = w;
    return hip_status(twell::launch_ffn_backward(a, static_cast<hipStream_t>(stream)));
}

size_t twell_ffn_decode_workspace_bytes(int32_t T, int32_t F, int32_t d, int32_t tile_w)
{
    if (T < 0 || T > twell::DEC_MAX_T || F <= 0 || d <= 0 || (tile_w != 32 && tile_w != 64 && tile_w != 128 &&
                                                             tile_w != 256) || F % tile_w != 0)
        return 0;
    return T <= twell::DEC2_MAX_T ? twell::decode_ws2_layout(nullptr, T, F, d).bytes
                                  : twell::decode_ws_layout(nullptr, T, F, tile_w, d).bytes;
}

int twell_ffn_decode(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                     const twell_hybrid_t *hy, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    TWELL_TRY(check_decode(x, wg_t, wu_t, wd, d, hy, y));
    if (hy->ell.T == 0)
        return TWELL_OK;
    if (!workspace)
        return TWELL_E_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return TWELL_E_ALIGN;
    const twell_t *h = &hy->ell;
    if (h->T > twell::DEC2_MAX_T) {
        const twell::DecodeWs w = twell::decode_ws_layout(workspace, h->T, h->F, h->tile_w, d);
        if (workspace_bytes < w.bytes)
            return TWELL_E_WORKSPACE;
        return launch_decode(x, wg_t, wu_t, wd, d, hy, y, w, static_cast<hipStream_t>(stream));
    }
    const twell::DecodeWs2 w = twell::decode_ws2_layout(workspace, h->T, h->F, d);
    if (workspace_bytes < w.bytes)
        return TWELL_E_WORKSPACE;
    return hip_status(twell::launch_decode2(x, wg_t, wu_t, wd, h->T, d, h->F, h->tile_w, h->cap, h->val, h->idx,
                                            h->cnt, hy->row_ovf, hy->ovf_rows, hy->n_ovf, hy->order, hy->max_ovf,
                                            hy->dense, y, w, static_cast<hipStream_t>(stream)));
}

int twell_ffn_decode_noalloc(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                             const twell_hybrid_t *hy, float *y, void *stream)
{
    TWELL_TRY(check_decode(x, wg_t, wu_t, wd, d, hy, y));
    if (hy->ell.T == 0)
        return TWELL_OK;
    const twell_t *h = &hy->ell;
    // the two-kernel organisation when its layout fits the scratch (its first
    // kernel clears the completion counter: nothing to clear here), else the
    // chunked kernels when theirs does
    const bool two = h->T <= twell::DEC2_MAX_T &&
                     twell::decode_ws2_layout(nullptr, h->T, h->F, d).bytes <= twell::DEC_STATIC_BYTES;
    if (!two && twell::decode_ws_layout(nullptr, h->T, h->F, h->tile_w, d).bytes > twell::DEC_STATIC_BYTES)
        return TWELL_E_SCRATCH;
    void *scratch = nullptr;
    TWELL_TRY(hip_status(twell::decode_static_workspace(&scratch)));
    if (two) {
        const twell::DecodeWs2 w = twell::decode_ws2_layout(scratch, h->T, h->F, d);
        return hip_status(twell::launch_decode2(x, wg_t, wu_t, wd, h->T, d, h->F, h->tile_w, h->cap, h->val, h->idx,
                                                h->cnt, hy->row_ovf, hy->ovf_rows, hy->n_ovf, hy->order, hy->max_ovf,
                                                hy->dense, y, w, static_cast<hipStream_t>(stream)));
    }
    const twell::DecodeWs w = twell::decode_ws_layout(scratch, h->T, h->F, h->tile_w, d);
    return launch_decode(x, wg_t, wu_t, wd, d, hy, y, w, static_cast<hipStream_t>(stream));
}

int twell_ffn_fused(const twell_t *h, const int32_t *order, const void *x, const void *wu_t, const void *wd,
                    int32_t d, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    TWELL_TRY(check_layout(h, d));
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_ptrs(h));
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wu_t));
    TWELL_TRY(check_mat(wd));
    TWELL_TRY(check_mat(y));
    if (reinterpret_cast<uintptr_t>(order) & 3u)
        return TWELL_E_ALIGN;
    const Ws w = ws_layout(h->T, h->F, h->tile_w, h->cap, 0, d, h->vdtype);
    TWELL_TRY(check_ws(workspace, workspace_bytes, w.bytes));
    return hip_status(twell::launch_ffn_fused(h->vdtype, h->cnt, h->val, h->idx, order, h->T, h->F, h->tile_w,
                                              h->cap, x, wu_t, wd, d, y, static_cast<char *>(workspace) + w.s_off,
                                              static_cast<hipStream_t>(stream)));
}

size_t twell_workspace_bytes(int32_t T, int32_t F, int32_t tile_w, int32_t cap, int32_t max_ovf, int32_t d,
                             int32_t vdtype)
{
    if (T < 0 || F <= 0 || d <= 0 || max_ovf < 0 || cap < 1 || (tile_w != 32 && tile_w != 64 && tile_w != 128 &&
                                                                 tile_w != 256) || F % tile_w != 0 ||
        (vdtype != TWELL_F32 && vdtype != TWELL_BF16))
        return 0;
    return ws_layout(T, F, tile_w, cap, max_ovf, d, vdtype).bytes;
}

int twell_ffn_overflow(const twell_hybrid_t *hy, const void *x, const void *wu_t, const void *wd, int32_t d,
                       float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *h = &hy->ell;
    TWELL_TRY(check_layout(h, d));
    TWELL_TRY(check_hybrid(hy));
    if (h->T == 0 || hy->max_ovf == 0)
        return TWELL_OK;
    TWELL_TRY(check_mat(x));
    TWELL_TRY(check_mat(wu_t));
    TWELL_TRY(check_mat(wd));
    TWELL_TRY(check_mat(y));
    const Ws w = ws_layout(hy, d);
    TWELL_TRY(check_ws(workspace, workspace_bytes, w.bytes));
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *pbuf = ws + w.p_off;
    float *part = w.splits > 1 ? reinterpret_cast<float *>(ws + w.part_off) : nullptr;
    TWELL_TRY(hip_status(twell::launch_gated_up(h->vdtype, x, h->T, wu_t, hy->ovf_rows, hy->n_ovf, hy->max_ovf, d, h->F,
                                                hy->dense, pbuf, s)));
    return hip_status(twell::launch_down(h->vdtype, pbuf, wd, hy->ovf_rows, hy->n_ovf, hy->max_ovf, h->F, d, y, part,
                                         w.splits, s));
}

int twell_ffn_hybrid(const twell_hybrid_t *hy, const void *x, const void *wu_t, const void *wd, int32_t d, float *y,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *h = &hy->ell;
    TWELL_TRY(check_layout(h, d));
    TWELL_TRY(check_hybrid(hy));
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_ws(workspace, workspace_bytes, ws_layout(hy, d).bytes));
    TWELL_TRY(twell_ffn_fused(h, hy->order, x, wu_t, wd, d, y, workspace, workspace_bytes, stream));
    return twell_ffn_overflow(hy, x, wu_t, wd, d, y, workspace, workspace_bytes, stream);
}

int twell_ffn_from_gate(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                        const twell_hybrid_t *hy, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    TWELL_TRY(check_layout(&hy->ell, d));
    TWELL_TRY(check_hybrid(hy));
    if (hy->ell.T == 0)
        return TWELL_OK;
    TWELL_TRY(check_layer(x, wg_t, wu_t, wd, d, hy, y, workspace, workspace_bytes));
    return launch_from_gate(x, wg_t, wu_t, wd, d, hy, y, workspace, static_cast<hipStream_t>(stream));
}

int twell_ffn_forward(const void *x, const void *wg_t, const void *wu_t, const void *wd, int32_t d,
                      const twell_hybrid_t *hy, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!hy)
        return TWELL_E_NULL;
    const twell_t *h = &hy->ell;
    TWELL_TRY(check_layout(h, d));
    TWELL_TRY(check_hybrid(hy));
    if (h->T == 0)
        return TWELL_OK;
    TWELL_TRY(check_layer(x, wg_t, wu_t, wd, d, hy, y, workspace, workspace_bytes));
    // every argument is checked: from here on only launches
    hipStream_t s = static_cast<hipStream_t>(stream);
    TWELL_TRY(hip_status(twell::launch_gate_twell(h->vdtype, x, wg_t, h->T, d, h->F, h->tile_w, h->cap, h->val,
                                                  h->idx, h->cnt, s)));
    return launch_from_gate(x, wg_t, wu_t, wd, d, hy, y, workspace, s);
}

}  // extern "C"
