// C ABI of libseqattn: argument validation, dispatch and launch on the
// caller's stream.  Declarations, semantics and passages: include/seqattn.h.
//
// Every check runs before the first HIP call, so each error return can be
// exercised on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/seqattn.h"
#include "common.h"

using namespace seqattn;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return SEQATTN_OK;
}

int esize(int32_t dt) { return dt == SEQATTN_BF16 ? 2 : 4; }

bool dtype_valid(int32_t dt) { return dt == SEQATTN_BF16 || dt == SEQATTN_F32; }

int64_t numel(const seqattn_tensor *t) { return t->b * t->h * t->n * t->d; }

constexpr int64_t kMaxRows = (int64_t)1 << 30;
constexpr int64_t kMaxBH = (int64_t)1 << 20;
constexpr int64_t kMaxStride = (int64_t)1 << 40;  // elements; keeps every extent in int64
constexpr int64_t kSplitCUs = 256;  // compute units of the GPU (a key-range split below one tile per CU)

// Structural checks of one descriptor: non-null, known dtype, non-negative
// dims within range, non-negative strides, 16-byte row alignment (rows, d>1).
int check_tensor(const seqattn_tensor *t, const char *name, bool is_lse)
{
    if (!t)
        return fail(SEQATTN_ERR_NULL, "%s: descriptor is NULL", name);
    if (!dtype_valid(t->dtype))
        return fail(SEQATTN_ERR_DTYPE, "%s: unknown dtype %d", name, (int)t->dtype);
    if (t->b < 0 || t->h < 0 || t->n < 0 || t->d < 0)
        return fail(SEQATTN_ERR_SHAPE, "%s: negative dimension", name);
    if (t->n >= kMaxRows || t->d >= kMaxRows || t->b >= kMaxBH || t->h >= kMaxBH ||
        t->b * t->h >= kMaxBH)
        return fail(SEQATTN_ERR_SHAPE, "%s: dimension too large", name);
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_n < 0)
        return fail(SEQATTN_ERR_STRIDE, "%s: negative stride", name);
    if (t->stride_b >= kMaxStride || t->stride_h >= kMaxStride || t->stride_n >= kMaxStride)
        return fail(SEQATTN_ERR_STRIDE, "%s: stride too large", name);
    if (numel(t) > 0) {
        // the byte span, which overlap tests and offsets below take in 64 bits
        const __int128 span = ((__int128)(t->b - 1) * t->stride_b +
                               (__int128)(t->h - 1) * t->stride_h +
                               (__int128)(t->n - 1) * t->stride_n + t->d) * esize(t->dtype);
        if (span >= ((__int128)1 << 56))
            return fail(SEQATTN_ERR_STRIDE, "%s: spans 2^56 bytes or more", name);
    }
    if (numel(t) > 0 && t->data == nullptr)
        return fail(SEQATTN_ERR_NULL, "%s: data pointer is NULL", name);
    if (is_lse) {
        if (t->dtype != SEQATTN_F32)
            return fail(SEQATTN_ERR_DTYPE, "%s: LSE must be fp32", name);
        if (t->d != 1)
            return fail(SEQATTN_ERR_SHAPE, "%s: LSE must have d == 1", name);
        if (((uintptr_t)t->data) % 4)
            return fail(SEQATTN_ERR_STRIDE, "%s: LSE data not 4-byte aligned", name);
        return SEQATTN_OK;
    }
    const int es = esize(t->dtype);
    if (numel(t) > 0) {
        if (((uintptr_t)t->data) % 16)
            return fail(SEQATTN_ERR_STRIDE, "%s: data not 16-byte aligned", name);
        if ((t->b > 1 && (t->stride_b * es) % 16) || (t->h > 1 && (t->stride_h * es) % 16) ||
            (t->n > 1 && (t->stride_n * es) % 16))
            return fail(SEQATTN_ERR_STRIDE, "%s: strides must be multiples of 16 bytes", name);
        if (t->n > 1 && t->stride_n < t->d)
            return fail(SEQATTN_ERR_STRIDE, "%s: rows overlap (stride_n < d)", name);
    }
    return SEQATTN_OK;
}

// Byte range [lo, hi) spanned by a descriptor (empty tensor -> empty range).
void extent(const seqattn_tensor *t, uintptr_t *lo, uintptr_t *hi)
{
    if (numel(t) == 0) {
        *lo = *hi = 0;
        return;
    }
    const int es = esize(t->dtype);
    const int64_t last = (t->b - 1) * t->stride_b + (t->h - 1) * t->stride_h +
                         (t->n - 1) * t->stride_n + t->d;
    *lo = (uintptr_t)t->data;
    *hi = (uintptr_t)t->data + (uintptr_t)last * es;
}

bool overlaps(const seqattn_tensor *a, const seqattn_tensor *b)
{
    uintptr_t al, ah, bl, bh;
    extent(a, &al, &ah);
    extent(b, &bl, &bh);
    if (al == ah || bl == bh)
        return false;
    return al < bh && bl < ah;
}

// An output's (b, h, n) rows must not overlap each other (else the writes of
// different rows race).  Sufficient test: with the dimensions of size > 1
// sorted by stride, each stride is at least the extent of the ones before.
int check_distinct_rows(const seqattn_tensor *t, const char *name)
{
    if (numel(t) == 0)
        return SEQATTN_OK;
    struct Dim {
        int64_t size, stride;
    } dims[3] = {{t->b, t->stride_b}, {t->h, t->stride_h}, {t->n, t->stride_n}};
    std::sort(dims, dims + 3, [](const Dim &x, const Dim &y) { return x.stride < y.stride; });
    int64_t extent = t->d;
    for (const Dim &dm : dims) {
        if (dm.size <= 1)
            continue;
        if (dm.stride < extent)
            return fail(SEQATTN_ERR_STRIDE, "%s: strides make rows overlap", name);
        extent = dm.stride * (dm.size - 1) + extent;
    }
    return SEQATTN_OK;
}

View view_of(const seqattn_tensor *t)
{
    View v;
    v.ptr = t->data;
    v.sb = t->stride_b;
    v.ss = 0;
    v.sh = t->stride_h;
    v.sn = t->stride_n;
    return v;
}

float pick_scale(float s, int64_t d) { return s > 0.f ? s : 1.0f / sqrtf((float)d); }

// Clamp delta into [-(Nq+1), Nk]; report non-causal when every key is visible
// to every query (delta >= Nk - 1).
void clamp_delta(int64_t delta, int64_t nq, int64_t nk, int *out, int *noncausal)
{
    if (delta == SEQATTN_NONCAUSAL || delta >= nk - 1) {
        *noncausal = 1;
        *out = (int)std::max<int64_t>(nk, 0);
        return;
    }
    *noncausal = 0;
    *out = (int)std::max<int64_t>(delta, -(nq + 1));
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(SEQATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Shared checks of (q, k, v) for the forward-style calls.
int check_qkv(const seqattn_tensor *q, const seqattn_tensor *k, const seqattn_tensor *v,
              bool same_len)
{
    int st;
    if ((st = check_tensor(q, "q", false)) || (st = check_tensor(k, "k", false)) ||
        (st = check_tensor(v, "v", false)))
        return st;
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(SEQATTN_ERR_DTYPE, "q, k, v must share one dtype");
    if (q->d != 64 && q->d != 128)
        return fail(SEQATTN_ERR_SHAPE, "head dim d=%lld not supported (64 or 128)",
                    (long long)q->d);
    if (k->d != q->d || v->d != q->d)
        return fail(SEQATTN_ERR_SHAPE, "q, k, v head dims differ");
    if (k->b != q->b || v->b != q->b)
        return fail(SEQATTN_ERR_SHAPE, "batch sizes differ");
    if (v->h != k->h || v->n != k->n)
        return fail(SEQATTN_ERR_SHAPE, "k and v shapes differ");
    if (k->h == 0 || q->h % k->h != 0)
        return fail(SEQATTN_ERR_SHAPE, "k->h (%lld) must divide q->h (%lld)",
                    (long long)k->h, (long long)q->h);
    if (same_len && k->n != q->n)
        return fail(SEQATTN_ERR_SHAPE, "q and k/v lengths differ");
    return SEQATTN_OK;
}

int check_out(const seqattn_tensor *o, const seqattn_tensor *lse, const seqattn_tensor *q,
              const seqattn_tensor *k, const seqattn_tensor *v)
{
    int st;
    if ((st = check_tensor(o, "o", false)) || (st = check_tensor(lse, "lse", true)))
        return st;
    if (o->b != q->b || o->h != q->h || o->n != q->n || o->d != q->d)
        return fail(SEQATTN_ERR_SHAPE, "o must be [B, Hq, Nq, d] like q");
    if (lse->b != q->b || lse->h != q->h || lse->n != q->n)
        return fail(SEQATTN_ERR_SHAPE, "lse must be [B, Hq, Nq, 1]");
    const seqattn_tensor *ins[3] = {q, k, v};
    for (const seqattn_tensor *in : ins)
        if (overlaps(o, in) || overlaps(lse, in))
            return fail(SEQATTN_ERR_ALIAS, "outputs overlap an input");
    if (overlaps(o, lse))
        return fail(SEQATTN_ERR_ALIAS, "o and lse overlap");
    if ((st = check_distinct_rows(o, "o")) || (st = check_distinct_rows(lse, "lse")))
        return st;
    return SEQATTN_OK;
}

hipStream_t stream_of(void *s) { return (hipStream_t)s; }

// Fixed device scratch of seqattn_attn_segment_bwd_noalloc: each GPU the
// library runs on holds one copy until the process ends.  In host code
// `scratch` names a host-side stand-in, so kernels get the device address
// that hipGetSymbolAddress returns for the device (kept per device).
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `s` (the current
// device for the null stream), looked up once per device with it current.
int scratch_for_stream(void *s, void **out)
{
    int dev = 0, cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return hip_status(e, "hipGetDevice");
    dev = cur;
    if (s) {
        e = hipStreamGetDevice(stream_of(s), &dev);
        if (e != hipSuccess)
            return hip_status(e, "hipStreamGetDevice");
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SEQATTN_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds",
                    dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return hip_status(e, "hipSetDevice");
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        if (e != hipSuccess)
            return hip_status(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SEQATTN_OK;
}

// The bf16 forward addresses one head's rows with 32-bit byte offsets
// (buffer loads, which also zero-fill rows past the end): each head's rows,
// plus the tile overrun of the last tile, must span less than 2 GiB.
int check_head_extent(const seqattn_tensor *t, const char *name, int64_t row_step)
{
    // rows < 2^31 + 2^29 and stride_n * esize < 2^42: the product fits in 128 bits
    const __int128 rows = (__int128)t->n + 512 * (__int128)row_step;
    if (rows * t->stride_n * esize(t->dtype) >= ((__int128)1 << 31))
        return fail(SEQATTN_ERR_UNSUPPORTED, "%s: one head spans >= 2 GiB", name);
    return SEQATTN_OK;
}

// The heads one launch of a dilated branch covers and their offset inside
// the segment.  Without head-dependent offsets (or with r = 1) it is every
// head at offset 0.  With them, query head h uses offset h mod r: the
// kernels apply it per head themselves (in_kernel), except in the backward
// with grouped KV heads, whose dK/dV workgroup serves query heads of
// different offsets; there each query head gets a launch of its own with
// its KV head.
struct HeadSel {
    int64_t qh, kh;   // first query head, first KV head
    int nq, nk;       // query heads, KV heads
    int64_t off;      // offset inside the segment (host-applied)
    bool in_kernel;   // the kernels shift head h by h mod r
};

std::vector<HeadSel> head_sels(bool shift, int64_t r, int Hq, int Hkv, bool kernel_ok)
{
    std::vector<HeadSel> out;
    if (!shift || r == 1) {
        out.push_back({0, 0, Hq, Hkv, 0, false});
    } else if (kernel_ok) {
        out.push_back({0, 0, Hq, Hkv, 0, true});
    } else {
        for (int64_t h = 0; h < Hq; ++h)
            out.push_back({h, (h * Hkv) / Hq, 1, 1, h % r, false});
    }
    return out;
}

// Key-range split of a segment forward whose 256-row query tiles are too
// few to fill the chip: each tile's visible keys are cut into nchunk equal
// parts (at least kv_chunk = 512 keys), computed by separate workgroups into
// fp32 partials and merged by their LSE.  A non-causal call with fewer tiles
// than compute units aims at one item per CU (all items equal).  A causal
// call with fewer than two tiles per CU aims at two items per CU: the parts
// shrink with their tiles, and heavy-first dispatch gives each CU one long
// and one short item (4 heads at 16K: 0.349 ms unsplit).  Decided from the
// shapes and causality alone (bf16, d = 128); the causal rule, which never
// takes fewer chunks, sizes the workspace.  Parts of at least 512 keys beat
// longer ones on the light tiles (8K tokens, 4 heads: 0.096 against 0.103 ms
// with 1024).
struct SegmentSplit {
    int nchunk = 1, kv_chunk = 0;
};

SegmentSplit segment_split(const seqattn_tensor *q, const seqattn_tensor *k, bool causal)
{
    constexpr int64_t kMinChunk = 512;
    SegmentSplit sp;
    if (!q || !k || q->dtype != SEQATTN_BF16 || q->d != 128 || k->n < 2 * kMinChunk)
        return sp;
    const int64_t tiles = q->b * q->h * ((q->n + 255) / 256);
    const int64_t items = causal ? 2 * kSplitCUs : kSplitCUs;
    if (tiles == 0 || tiles >= items)
        return sp;
    const int64_t want = std::min<int64_t>((items + tiles - 1) / tiles, 8);
    // the longest tile's parts: at least 1024 keys from 4096 keys on (eight
    // parts of 512 at 4K tokens and 4 heads took 0.057 ms, four 0.044)
    const int64_t cap = k->n / (k->n >= 4096 ? 1024 : kMinChunk);
    sp.nchunk = (int)std::min<int64_t>(want, cap);
    sp.kv_chunk = (int)kMinChunk;
    if (sp.nchunk < 2)
        sp = SegmentSplit();
    return sp;
}

size_t segment_split_bytes(const seqattn_tensor *q, const SegmentSplit &sp)
{
    if (sp.nchunk < 2)
        return 0;
    return (size_t)sp.nchunk * (size_t)(q->b * q->h * q->n) * (size_t)(q->d + 1) * sizeof(float);
}

int segment_fwd(const seqattn_tensor *q, const seqattn_tensor *k, const seqattn_tensor *v,
                int64_t causal_offset, float softmax_scale, uint32_t flags, seqattn_tensor *o,
                seqattn_tensor *lse, void *workspace, size_t workspace_bytes, bool may_split,
                void *hip_stream)
{
    int st;
    if ((st = check_qkv(q, k, v, false)) || (st = check_out(o, lse, q, k, v)))
        return st;
    if (flags & ~SEQATTN_ACCUMULATE)
        return fail(SEQATTN_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    const bool acc = flags & SEQATTN_ACCUMULATE;
    if ((acc || q->dtype == SEQATTN_F32) && o->dtype != SEQATTN_F32)
        return fail(SEQATTN_ERR_DTYPE, "o must be fp32 (accumulate or fp32 inputs)");
    if (q->dtype == SEQATTN_BF16 &&
        ((st = check_head_extent(q, "q", 1)) || (st = check_head_extent(k, "k", 1)) ||
         (st = check_head_extent(v, "v", 1))))
        return st;

    FwdParams p;
    p.q = view_of(q);
    p.k = view_of(k);
    p.v = view_of(v);
    p.o = view_of(o);
    p.lse = view_of(lse);
    p.B = (int)q->b;
    p.S = 1;
    p.Hq = (int)q->h;
    p.Hkv = (int)k->h;
    p.Nq = (int)q->n;
    p.Nk = (int)k->n;
    clamp_delta(causal_offset, q->n, k->n, &p.delta, &p.noncausal);
    p.scale = pick_scale(softmax_scale, q->d);
    p.accumulate = acc ? 1 : 0;
    p.o_f32 = o->dtype == SEQATTN_F32;
    if (p.Nq == 0 || p.B == 0 || p.Hq == 0)
        return ok();
    if (p.Nk == 0) {
        if (acc)
            return ok();
        return hip_status(launch_fill_empty(p.o, p.lse, p.B, 1, p.Hq, p.Nq, (int)q->d,
                                            p.o_f32, stream_of(hip_stream)),
                          "fill_empty");
    }
    const SegmentSplit sp =
        may_split && !acc ? segment_split(q, k, !p.noncausal) : SegmentSplit();
    if (sp.nchunk > 1) {
        const size_t need = segment_split_bytes(q, sp);
        if (!workspace || workspace_bytes < need)
            return fail(SEQATTN_ERR_WORKSPACE, "need %zu bytes of workspace", need);
        if ((uintptr_t)workspace % 16)
            return fail(SEQATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        const uintptr_t wl = (uintptr_t)workspace, wh = wl + need;
        const seqattn_tensor *all[5] = {q, k, v, o, lse};
        for (const seqattn_tensor *t : all) {
            uintptr_t tl, th;
            extent(t, &tl, &th);
            if (tl != th && tl < wh && wl < th)
                return fail(SEQATTN_ERR_ALIAS, "workspace overlaps a tensor");
        }
        // partials: O [nchunk][B][Hq][Nq][d], then LSE [nchunk][B][Hq][Nq], fp32
        const int64_t bhn = (int64_t)p.B * p.Hq * p.Nq;
        float *po = (float *)workspace;
        float *pl = po + sp.nchunk * bhn * q->d;
        FwdParams s = p;
        s.o.ptr = po;
        s.o.sb = (int64_t)p.Hq * p.Nq * q->d;
        s.o.ss = 0;
        s.o.sh = (int64_t)p.Nq * q->d;
        s.o.sn = q->d;
        s.lse.ptr = pl;
        s.lse.sb = (int64_t)p.Hq * p.Nq;
        s.lse.ss = 0;
        s.lse.sh = p.Nq;
        s.lse.sn = 1;
        s.o_f32 = 1;
        s.kv_chunk = sp.kv_chunk;
        s.nchunk = sp.nchunk;
        s.o_chunk = bhn * q->d;
        s.l_chunk = bhn;
        hipError_t e = launch_fwd_bf16(s, (int)q->d, stream_of(hip_stream));
        if (e != hipSuccess)
            return hip_status(e, "attn_segment_fwd launch");
        ChunkMergeParams m;
        m.o = p.o;
        m.lse = p.lse;
        m.po = po;
        m.pl = pl;
        m.B = p.B;
        m.H = p.Hq;
        m.N = p.Nq;
        m.d = (int)q->d;
        m.Nk = p.Nk;
        m.delta = p.delta;
        m.noncausal = p.noncausal;
        m.tile_rows = 256;
        m.kv_chunk = sp.kv_chunk;
        m.nchunk = sp.nchunk;
        m.o_f32 = p.o_f32;
        return hip_status(launch_chunk_merge(m, stream_of(hip_stream)), "chunk merge launch");
    }
    const hipError_t e = q->dtype == SEQATTN_BF16
                             ? launch_fwd_bf16(p, (int)q->d, stream_of(hip_stream))
                             : launch_fwd_f32(p, (int)q->d, stream_of(hip_stream));
    return hip_status(e, "attn_segment_fwd launch");
}

}  // namespace

extern "C" {

int seqattn_version(void) { return SEQATTN_VERSION; }

const char *seqattn_status_string(int status)
{
    switch (status) {
    case SEQATTN_OK: return "ok";
    case SEQATTN_ERR_NULL: return "null pointer";
    case SEQATTN_ERR_DTYPE: return "unsupported or mismatched dtype";
    case SEQATTN_ERR_SHAPE: return "invalid shape";
    case SEQATTN_ERR_STRIDE: return "invalid stride or alignment";
    case SEQATTN_ERR_ALIAS: return "output aliases an input";
    case SEQATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case SEQATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SEQATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *seqattn_last_error(void) { return g_err; }

int seqattn_attn_segment_fwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, int64_t causal_offset,
                             float softmax_scale, uint32_t flags, seqattn_tensor *o,
                             seqattn_tensor *lse, void *hip_stream)
{
    return segment_fwd(q, k, v, causal_offset, softmax_scale, flags, o, lse, nullptr, 0, false,
                       hip_stream);
}

int seqattn_attn_segment_fwd_ws(const seqattn_tensor *q, const seqattn_tensor *k,
                                const seqattn_tensor *v, int64_t causal_offset,
                                float softmax_scale, uint32_t flags, seqattn_tensor *o,
                                seqattn_tensor *lse, void *workspace, size_t workspace_bytes,
                                void *hip_stream)
{
    return segment_fwd(q, k, v, causal_offset, softmax_scale, flags, o, lse, workspace,
                       workspace_bytes, true, hip_stream);
}

int seqattn_lse_merge(seqattn_tensor *o_acc, seqattn_tensor *lse_acc,
                      const seqattn_tensor *o_b, const seqattn_tensor *lse_b,
                      void *hip_stream)
{
    int st;
    if ((st = check_tensor(o_acc, "o_acc", false)) ||
        (st = check_tensor(lse_acc, "lse_acc", true)) ||
        (st = check_tensor(o_b, "o_b", false)) || (st = check_tensor(lse_b, "lse_b", true)))
        return st;
    if (o_acc->dtype != SEQATTN_F32)
        return fail(SEQATTN_ERR_DTYPE, "o_acc must be fp32");
    if (o_acc->d % 8 != 0 || o_acc->d == 0)
        return fail(SEQATTN_ERR_SHAPE, "d must be a positive multiple of 8");
    if (o_b->b != o_acc->b || o_b->h != o_acc->h || o_b->n != o_acc->n || o_b->d != o_acc->d)
        return fail(SEQATTN_ERR_SHAPE, "o_b shape differs from o_acc");
    const seqattn_tensor *ls[2] = {lse_acc, lse_b};
    for (const seqattn_tensor *l : ls)
        if (l->b != o_acc->b || l->h != o_acc->h || l->n != o_acc->n)
            return fail(SEQATTN_ERR_SHAPE, "lse shape must be [B, H, N, 1]");
    if (overlaps(o_acc, o_b) || overlaps(o_acc, lse_b) || overlaps(lse_acc, o_b) ||
        overlaps(lse_acc, lse_b) || overlaps(o_acc, lse_acc))
        return fail(SEQATTN_ERR_ALIAS, "accumulator overlaps the merged partial");
    if ((st = check_distinct_rows(o_acc, "o_acc")) || (st = check_distinct_rows(lse_acc, "lse_acc")))
        return st;
    MergeParams p;
    p.oa = view_of(o_acc);
    p.la = view_of(lse_acc);
    p.ob = view_of(o_b);
    p.lb = view_of(lse_b);
    p.B = (int)o_acc->b;
    p.H = (int)o_acc->h;
    p.N = (int)o_acc->n;
    p.d = (int)o_acc->d;
    p.ob_f32 = o_b->dtype == SEQATTN_F32;
    return hip_status(launch_lse_merge(p, stream_of(hip_stream)), "lse_merge launch");
}

size_t seqattn_workspace_size(int op, const seqattn_tensor *q, const seqattn_tensor *k,
                              int32_t n_branches)
{
    (void)n_branches;
    if (!q)
        return 0;
    switch (op) {
    case SEQATTN_OP_SEGMENT_FWD:
        // fp32 partials of a key-range split (seqattn_attn_segment_fwd_ws)
        return segment_split_bytes(q, segment_split(q, k, true));
    case SEQATTN_OP_DILATED_FWD:
        // fp32 accumulator when the output o (passed as `k`) is bf16
        if (k && k->dtype == SEQATTN_BF16)
            return (size_t)(q->b * q->h * q->n * q->d) * sizeof(float);
        return 0;
    case SEQATTN_OP_SEGMENT_BWD:
    case SEQATTN_OP_DILATED_BWD:
        // D_i = sum_c dO_ic O_ic per query row
        return (size_t)(q->b * q->h * q->n) * sizeof(float);
    default:
        return 0;
    }
}

int seqattn_dilated_attn_fwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, const int64_t *segment_lengths,
                             const int64_t *dilations, int32_t n_branches,
                             float softmax_scale, uint32_t flags, seqattn_tensor *o,
                             seqattn_tensor *lse, void *workspace, size_t workspace_bytes,
                             void *hip_stream)
{
    int st;
    if ((st = check_qkv(q, k, v, true)) || (st = check_out(o, lse, q, k, v)))
        return st;
    if (q->dtype != SEQATTN_BF16)
        return fail(SEQATTN_ERR_DTYPE, "dilated attention takes bf16 q/k/v");
    if (!segment_lengths || !dilations)
        return fail(SEQATTN_ERR_NULL, "segment_lengths / dilations are NULL");
    if (n_branches < 1 || n_branches > 64)
        return fail(SEQATTN_ERR_SHAPE, "n_branches must be in [1, 64]");
    if (flags & ~(SEQATTN_CAUSAL | SEQATTN_HEAD_SHIFT))
        return fail(SEQATTN_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    for (int i = 0; i < n_branches; ++i)
        if (segment_lengths[i] < 1 || dilations[i] < 1 || segment_lengths[i] >= kMaxRows ||
            dilations[i] >= kMaxRows)
            return fail(SEQATTN_ERR_SHAPE, "branch %d: w and r must be >= 1", i);
    int64_t rmax = 1;
    for (int i = 0; i < n_branches; ++i)
        rmax = std::max<int64_t>(rmax, dilations[i]);
    if ((st = check_head_extent(q, "q", rmax)) || (st = check_head_extent(k, "k", rmax)) ||
        (st = check_head_extent(v, "v", rmax)))
        return st;
    const bool o_bf16 = o->dtype == SEQATTN_BF16;
    const size_t need = seqattn_workspace_size(SEQATTN_OP_DILATED_FWD, q, o, n_branches);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(SEQATTN_ERR_WORKSPACE, "need %zu bytes of workspace", need);
        if ((uintptr_t)workspace % 16)
            return fail(SEQATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    }
    const int B = (int)q->b, Hq = (int)q->h, N = (int)q->n, d = (int)q->d;
    if (B == 0 || Hq == 0 || N == 0)
        return ok();
    hipStream_t s = stream_of(hip_stream);

    // The accumulator: o itself when fp32, else the fp32 workspace [B,Hq,N,d].
    View acc = view_of(o);
    if (o_bf16) {
        acc.ptr = workspace;
        acc.sb = (int64_t)Hq * N * d;
        acc.sh = (int64_t)N * d;
        acc.sn = d;
    }
    View lsev = view_of(lse);
    const bool causal = flags & SEQATTN_CAUSAL;
    const float scale = pick_scale(softmax_scale, d);

    // A first branch with r = 1 selects every position: it can overwrite the
    // accumulator instead of merging into an initialised one.
    const bool first_writes = dilations[0] == 1;
    if (!first_writes) {
        hipError_t e = launch_fill_empty(acc, lsev, B, 1, Hq, N, d, 1, s);
        if (e != hipSuccess)
            return hip_status(e, "dilated init");
    }
    const bool shift = flags & SEQATTN_HEAD_SHIFT;
    for (int i = 0; i < n_branches; ++i) {
        const int64_t w = std::min<int64_t>(segment_lengths[i], N), r = dilations[i];
        const int64_t nfull = N / w, tail = N % w;
        for (const HeadSel &hs : head_sels(shift, r, Hq, (int)k->h, true))
        for (int part = 0; part < 2; ++part) {
            const int64_t nseg = part == 0 ? nfull : (tail > 0 ? 1 : 0);
            const int64_t seglen = part == 0 ? w : tail;
            if (nseg == 0 || seglen <= hs.off)
                continue;
            const int64_t base = (part == 0 ? 0 : nfull * w) + hs.off;  // first selected row
            const int64_t rows = (seglen - hs.off + r - 1) / r;        // selected rows per segment
            // [B][segment][head][selected row] view of the heads hs covers
            auto sub = [&](View vv, int64_t es, int64_t head0) {
                View x = vv;
                x.ptr = (const char *)vv.ptr + (base * vv.sn + head0 * vv.sh) * es;
                x.ss = w * vv.sn;
                x.sn = r * vv.sn;
                return x;
            };
            FwdParams p;
            p.q = sub(view_of(q), 2, hs.qh);
            p.k = sub(view_of(k), 2, hs.kh);
            p.v = sub(view_of(v), 2, hs.kh);
            p.o = sub(acc, 4, hs.qh);
            p.lse = sub(lsev, 4, hs.qh);
            p.B = B;
            p.S = (int)nseg;
            p.Hq = hs.nq;
            p.Hkv = hs.nk;
            p.Nq = p.Nk = (int)rows;
            clamp_delta(causal ? 0 : SEQATTN_NONCAUSAL, rows, rows, &p.delta, &p.noncausal);
            p.scale = scale;
            p.accumulate = (i == 0 && first_writes) ? 0 : 1;
            p.o_f32 = 1;
            p.hs_r = hs.in_kernel ? (int)r : 0;
            p.hs_len = (int)seglen;
            hipError_t e = launch_fwd_bf16(p, d, s);
            if (e != hipSuccess)
                return hip_status(e, "dilated branch launch");
        }
    }
    if (o_bf16) {
        hipError_t e = launch_cast_bf16(acc, view_of(o), B, Hq, N, d, s);
        if (e != hipSuccess)
            return hip_status(e, "dilated cast");
    }
    return ok();
}

}  // extern "C"

namespace {

// The segment backward; D goes to the caller's workspace, or with
// use_scratch to the fixed per-device scratch (no workspace argument).
int segment_bwd(const seqattn_tensor *q, const seqattn_tensor *k, const seqattn_tensor *v,
                const seqattn_tensor *o, const seqattn_tensor *lse, const seqattn_tensor *d_o,
                int64_t causal_offset, float softmax_scale, uint32_t flags,
                seqattn_tensor *dq, seqattn_tensor *dk, seqattn_tensor *dv, void *workspace,
                size_t workspace_bytes, bool use_scratch, void *hip_stream)
{
    int st;
    if ((st = check_qkv(q, k, v, false)))
        return st;
    if ((st = check_tensor(o, "o", false)) || (st = check_tensor(lse, "lse", true)) ||
        (st = check_tensor(d_o, "d_o", false)) || (st = check_tensor(dq, "dq", false)) ||
        (st = check_tensor(dk, "dk", false)) || (st = check_tensor(dv, "dv", false)))
        return st;
    if (q->dtype != SEQATTN_BF16)
        return fail(SEQATTN_ERR_UNSUPPORTED, "backward takes bf16 q/k/v");
    if (d_o->dtype != SEQATTN_BF16)
        return fail(SEQATTN_ERR_DTYPE, "d_o must be bf16");
    // the dQ kernel also reads K and V tiles with 32-bit offsets
    if ((st = check_head_extent(q, "q", 1)) || (st = check_head_extent(d_o, "d_o", 1)) ||
        (st = check_head_extent(k, "k", 1)) || (st = check_head_extent(v, "v", 1)))
        return st;
    if (dq->dtype != SEQATTN_F32)
        return fail(SEQATTN_ERR_DTYPE, "dq must be fp32 (accumulated)");
    if (flags & ~SEQATTN_ACCUMULATE)
        return fail(SEQATTN_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    const bool acc_kv = flags & SEQATTN_ACCUMULATE;
    if (acc_kv && (dk->dtype != SEQATTN_F32 || dv->dtype != SEQATTN_F32))
        return fail(SEQATTN_ERR_DTYPE, "dk, dv must be fp32 with SEQATTN_ACCUMULATE");
    const seqattn_tensor *qlike[3] = {o, d_o, dq};
    for (const seqattn_tensor *t : qlike)
        if (t->b != q->b || t->h != q->h || t->n != q->n || t->d != q->d)
            return fail(SEQATTN_ERR_SHAPE, "o, d_o, dq must be [B, Hq, Nq, d]");
    if (lse->b != q->b || lse->h != q->h || lse->n != q->n)
        return fail(SEQATTN_ERR_SHAPE, "lse must be [B, Hq, Nq, 1]");
    const seqattn_tensor *klike[2] = {dk, dv};
    for (const seqattn_tensor *t : klike)
        if (t->b != k->b || t->h != k->h || t->n != k->n || t->d != k->d)
            return fail(SEQATTN_ERR_SHAPE, "dk, dv must be [B, Hkv, Nk, d]");
    const seqattn_tensor *ins[6] = {q, k, v, o, lse, d_o};
    const seqattn_tensor *outs[3] = {dq, dk, dv};
    for (const seqattn_tensor *a : outs) {
        for (const seqattn_tensor *b : ins)
            if (overlaps(a, b))
                return fail(SEQATTN_ERR_ALIAS, "a gradient overlaps an input");
        for (const seqattn_tensor *b : outs)
            if (a != b && overlaps(a, b))
                return fail(SEQATTN_ERR_ALIAS, "gradients overlap each other");
        if ((st = check_distinct_rows(a, "gradient")))
            return st;
    }
    const size_t need = seqattn_workspace_size(SEQATTN_OP_SEGMENT_BWD, q, k, 0);
    if (use_scratch) {
        if (need > kScratchBytes)
            return fail(SEQATTN_ERR_WORKSPACE,
                        "needs %zu bytes of scratch, above the fixed %zu (B*Hq*Nq <= %zu)",
                        need, kScratchBytes, kScratchBytes / sizeof(float));
        workspace = nullptr;
        const bool empty = q->b == 0 || k->h == 0 || (k->n == 0 && q->n == 0);
        if (need > 0 && !empty && (st = scratch_for_stream(hip_stream, &workspace)))
            return st;
    } else {
        if (need > 0 && (!workspace || workspace_bytes < need))
            return fail(SEQATTN_ERR_WORKSPACE, "need %zu bytes of workspace", need);
        if (workspace && (uintptr_t)workspace % 16)
            return fail(SEQATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    }

    BwdParams p;
    p.q = view_of(q);
    p.k = view_of(k);
    p.v = view_of(v);
    p.o = view_of(o);
    p.lse = view_of(lse);
    p.dout = view_of(d_o);
    p.dq = view_of(dq);
    p.dk = view_of(dk);
    p.dv = view_of(dv);
    p.dvec.ptr = workspace;
    p.dvec.sb = q->h * q->n;
    p.dvec.ss = 0;
    p.dvec.sh = q->n;
    p.dvec.sn = 1;
    p.B = (int)q->b;
    p.S = 1;
    p.Hq = (int)q->h;
    p.Hkv = (int)k->h;
    p.Nq = (int)q->n;
    p.Nk = (int)k->n;
    p.d = (int)q->d;
    clamp_delta(causal_offset, q->n, k->n, &p.delta, &p.noncausal);
    p.scale = pick_scale(softmax_scale, q->d);
    p.o_f32 = o->dtype == SEQATTN_F32;
    p.dk_f32 = dk->dtype == SEQATTN_F32;
    p.dv_f32 = dv->dtype == SEQATTN_F32;
    p.acc_kv = acc_kv ? 1 : 0;
    if (p.B == 0 || p.Hkv == 0 || (p.Nk == 0 && p.Nq == 0))
        return ok();
    hipError_t e = launch_bwd_prep(p, stream_of(hip_stream));
    if (e != hipSuccess)
        return hip_status(e, "attn_segment_bwd prep launch");
    return hip_status(launch_bwd_bf16(p, stream_of(hip_stream)), "attn_segment_bwd launch");
}

}  // namespace

extern "C" {

int seqattn_attn_segment_bwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, const seqattn_tensor *o,
                             const seqattn_tensor *lse, const seqattn_tensor *d_o,
                             int64_t causal_offset, float softmax_scale, uint32_t flags,
                             seqattn_tensor *dq, seqattn_tensor *dk, seqattn_tensor *dv,
                             void *workspace, size_t workspace_bytes, void *hip_stream)
{
    return segment_bwd(q, k, v, o, lse, d_o, causal_offset, softmax_scale, flags, dq, dk, dv,
                       workspace, workspace_bytes, false, hip_stream);
}

int seqattn_attn_segment_bwd_noalloc(const seqattn_tensor *q, const seqattn_tensor *k,
                                     const seqattn_tensor *v, const seqattn_tensor *o,
                                     const seqattn_tensor *lse, const seqattn_tensor *d_o,
                                     int64_t causal_offset, float softmax_scale,
                                     uint32_t flags, seqattn_tensor *dq, seqattn_tensor *dk,
                                     seqattn_tensor *dv, void *hip_stream)
{
    return segment_bwd(q, k, v, o, lse, d_o, causal_offset, softmax_scale, flags, dq, dk, dv,
                       nullptr, 0, true, hip_stream);
}

int seqattn_dilated_attn_bwd(const seqattn_tensor *q, const seqattn_tensor *k,
                             const seqattn_tensor *v, const seqattn_tensor *o,
                             const seqattn_tensor *lse, const seqattn_tensor *d_o,
                             const int64_t *segment_lengths, const int64_t *dilations,
                             int32_t n_branches, float softmax_scale, uint32_t flags,
                             seqattn_tensor *dq, seqattn_tensor *dk, seqattn_tensor *dv,
                             void *workspace, size_t workspace_bytes, void *hip_stream)
{
    int st;
    if ((st = check_qkv(q, k, v, true)))
        return st;
    if ((st = check_tensor(o, "o", false)) || (st = check_tensor(lse, "lse", true)) ||
        (st = check_tensor(d_o, "d_o", false)) || (st = check_tensor(dq, "dq", false)) ||
        (st = check_tensor(dk, "dk", false)) || (st = check_tensor(dv, "dv", false)))
        return st;
    if (q->dtype != SEQATTN_BF16)
        return fail(SEQATTN_ERR_DTYPE, "dilated attention takes bf16 q/k/v");
    if (d_o->dtype != SEQATTN_BF16)
        return fail(SEQATTN_ERR_DTYPE, "d_o must be bf16");
    if (dq->dtype != SEQATTN_F32 || dk->dtype != SEQATTN_F32 || dv->dtype != SEQATTN_F32)
        return fail(SEQATTN_ERR_DTYPE, "dq, dk, dv must be fp32");
    if (!segment_lengths || !dilations)
        return fail(SEQATTN_ERR_NULL, "segment_lengths / dilations are NULL");
    if (n_branches < 1 || n_branches > 64)
        return fail(SEQATTN_ERR_SHAPE, "n_branches must be in [1, 64]");
    if (flags & ~(SEQATTN_CAUSAL | SEQATTN_HEAD_SHIFT))
        return fail(SEQATTN_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    for (int i = 0; i < n_branches; ++i)
        if (segment_lengths[i] < 1 || dilations[i] < 1 || segment_lengths[i] >= kMaxRows ||
            dilations[i] >= kMaxRows)
            return fail(SEQATTN_ERR_SHAPE, "branch %d: w and r must be >= 1", i);
    const seqattn_tensor *qlike[3] = {o, d_o, dq};
    for (const seqattn_tensor *t : qlike)
        if (t->b != q->b || t->h != q->h || t->n != q->n || t->d != q->d)
            return fail(SEQATTN_ERR_SHAPE, "o, d_o, dq must be [B, Hq, N, d]");
    if (lse->b != q->b || lse->h != q->h || lse->n != q->n)
        return fail(SEQATTN_ERR_SHAPE, "lse must be [B, Hq, N, 1]");
    const seqattn_tensor *klike[2] = {dk, dv};
    for (const seqattn_tensor *t : klike)
        if (t->b != k->b || t->h != k->h || t->n != k->n || t->d != k->d)
            return fail(SEQATTN_ERR_SHAPE, "dk, dv must be [B, Hkv, N, d]");
    const seqattn_tensor *ins[6] = {q, k, v, o, lse, d_o};
    const seqattn_tensor *outs[3] = {dq, dk, dv};
    for (const seqattn_tensor *a : outs) {
        for (const seqattn_tensor *b : ins)
            if (overlaps(a, b))
                return fail(SEQATTN_ERR_ALIAS, "a gradient overlaps an input");
        for (const seqattn_tensor *b : outs)
            if (a != b && overlaps(a, b))
                return fail(SEQATTN_ERR_ALIAS, "gradients overlap each other");
        if ((st = check_distinct_rows(a, "gradient")))
            return st;
    }
    int64_t rmax = 1;
    for (int i = 0; i < n_branches; ++i)
        rmax = std::max<int64_t>(rmax, dilations[i]);
    if ((st = check_head_extent(q, "q", rmax)) || (st = check_head_extent(k, "k", rmax)) ||
        (st = check_head_extent(v, "v", rmax)) || (st = check_head_extent(d_o, "d_o", rmax)))
        return st;
    const size_t need = seqattn_workspace_size(SEQATTN_OP_DILATED_BWD, q, k, n_branches);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(SEQATTN_ERR_WORKSPACE, "need %zu bytes of workspace", need);
    if (workspace && (uintptr_t)workspace % 16)
        return fail(SEQATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    const int B = (int)q->b, Hq = (int)q->h, Hkv = (int)k->h, N = (int)q->n, d = (int)q->d;
    if (B == 0 || N == 0)
        return ok();
    hipStream_t s = stream_of(hip_stream);
    const bool causal = flags & SEQATTN_CAUSAL;

    // D over every query row, from the merged (all-branch) O and dO.
    BwdParams base;
    base.q = view_of(q);
    base.k = view_of(k);
    base.v = view_of(v);
    base.o = view_of(o);
    base.lse = view_of(lse);
    base.dout = view_of(d_o);
    base.dq = view_of(dq);
    base.dk = view_of(dk);
    base.dv = view_of(dv);
    base.dvec.ptr = workspace;
    base.dvec.sb = (int64_t)Hq * N;
    base.dvec.ss = 0;
    base.dvec.sh = N;
    base.dvec.sn = 1;
    base.B = B;
    base.S = 1;
    base.Hq = Hq;
    base.Hkv = Hkv;
    base.Nq = base.Nk = N;
    base.d = d;
    base.delta = 0;
    base.noncausal = 1;
    base.scale = pick_scale(softmax_scale, d);
    base.o_f32 = o->dtype == SEQATTN_F32;
    base.dk_f32 = base.dv_f32 = 1;
    base.acc_kv = 0;
    hipError_t e = launch_bwd_prep(base, s);
    if (e != hipSuccess)
        return hip_status(e, "dilated bwd prep launch");

    // A first branch with r = 1 touches every key row: it writes dK/dV, every
    // later branch adds to them.  Otherwise they start from zero.
    const bool first_writes = dilations[0] == 1;
    if (!first_writes) {
        if ((e = launch_zero_f32(base.dk, B, Hkv, N, d, s)) != hipSuccess ||
            (e = launch_zero_f32(base.dv, B, Hkv, N, d, s)) != hipSuccess)
            return hip_status(e, "dilated bwd init");
    }
    const bool shift = flags & SEQATTN_HEAD_SHIFT;
    for (int i = 0; i < n_branches; ++i) {
        const int64_t w = std::min<int64_t>(segment_lengths[i], N), r = dilations[i];
        const int64_t nfull = N / w, tail = N % w;
        for (const HeadSel &hs : head_sels(shift, r, Hq, Hkv, Hq == Hkv))
        for (int part = 0; part < 2; ++part) {
            const int64_t nseg = part == 0 ? nfull : (tail > 0 ? 1 : 0);
            const int64_t seglen = part == 0 ? w : tail;
            if (nseg == 0 || seglen <= hs.off)
                continue;
            const int64_t row0 = (part == 0 ? 0 : nfull * w) + hs.off;
            const int64_t rows = (seglen - hs.off + r - 1) / r;
            // Branch i's selected rows of each segment for the heads hs
            // covers, as a [B][seg][H][rows] view.
            auto sub = [&](View vv, int64_t es, int64_t head0) {
                View x = vv;
                x.ptr = (const char *)vv.ptr + (row0 * vv.sn + head0 * vv.sh) * es;
                x.ss = w * vv.sn;
                x.sn = r * vv.sn;
                return x;
            };
            BwdParams p = base;
            p.q = sub(base.q, 2, hs.qh);
            p.k = sub(base.k, 2, hs.kh);
            p.v = sub(base.v, 2, hs.kh);
            p.lse = sub(base.lse, 4, hs.qh);
            p.dout = sub(base.dout, 2, hs.qh);
            p.dq = sub(base.dq, 4, hs.qh);
            p.dk = sub(base.dk, 4, hs.kh);
            p.dv = sub(base.dv, 4, hs.kh);
            p.dvec = sub(base.dvec, 4, hs.qh);
            p.Hq = hs.nq;
            p.Hkv = hs.nk;
            p.S = (int)nseg;
            p.Nq = p.Nk = (int)rows;
            clamp_delta(causal ? 0 : SEQATTN_NONCAUSAL, rows, rows, &p.delta, &p.noncausal);
            p.acc_kv = (i == 0 && first_writes) ? 0 : 1;
            p.hs_r = hs.in_kernel ? (int)r : 0;
            p.hs_len = (int)seglen;
            if ((e = launch_bwd_bf16(p, s)) != hipSuccess)
                return hip_status(e, "dilated bwd branch launch");
        }
    }
    return ok();
}

int seqattn_head_relayout(const seqattn_tensor *src, seqattn_tensor *dst, void *hip_stream)
{
    int st;
    if ((st = check_tensor(src, "src", false)) || (st = check_tensor(dst, "dst", false)))
        return st;
    if (src->dtype != dst->dtype)
        return fail(SEQATTN_ERR_DTYPE, "src and dst dtypes differ");
    if (src->n != dst->n || src->d != dst->d || src->b * src->h != dst->b * dst->h)
        return fail(SEQATTN_ERR_SHAPE, "src and dst must hold the same b*h heads of n rows of d");
    const int64_t row_bytes = src->d * esize(src->dtype);
    if (row_bytes % 16)
        return fail(SEQATTN_ERR_SHAPE, "d * element size must be a multiple of 16 bytes");
    const int64_t heads = src->b * src->h;
    if (heads == 0 || src->n == 0 || src->d == 0)
        return ok();
    if ((row_bytes / 16) * heads * src->n >= ((int64_t)1 << 31))
        return fail(SEQATTN_ERR_UNSUPPORTED, "more than 2^31 16-byte units in one call");
    if (src->h == 0 || dst->h == 0)
        return fail(SEQATTN_ERR_SHAPE, "h must be positive");
    if (overlaps(src, dst))
        return fail(SEQATTN_ERR_ALIAS, "dst overlaps src");
    if ((st = check_distinct_rows(dst, "dst")))
        return st;
    const int es = esize(src->dtype);
    RelayoutParams p;
    p.src = (const char *)src->data;
    p.dst = (char *)dst->data;
    p.s_sb = src->stride_b * es;
    p.s_sh = src->stride_h * es;
    p.s_sn = src->stride_n * es;
    p.d_sb = dst->stride_b * es;
    p.d_sh = dst->stride_h * es;
    p.d_sn = dst->stride_n * es;
    p.src_h = (uint32_t)src->h;
    p.dst_h = (uint32_t)dst->h;
    p.F = (uint32_t)heads;
    p.N = (uint32_t)src->n;
    p.units = (uint32_t)(row_bytes / 16);
    // lanes walk the source's faster-moving of (head, row)
    const int64_t src_head_stride = src->h > 1 ? src->stride_h : src->stride_b;
    p.head_fast = (heads > 1 && src->n > 1 && src_head_stride < src->stride_n) ? 1 : 0;
    return hip_status(launch_head_relayout(p, stream_of(hip_stream)), "head_relayout launch");
}

}  // extern "C"
