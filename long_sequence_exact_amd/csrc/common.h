// Internal parameter blocks shared by the ABI layer and the HIP kernels.
// Not part of the public C ABI (include/seqattn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seqattn {

// One strided view [batch][seg][head][row][d] of a tensor (element strides;
// d contiguous).  `seg` is an extra batch-like dimension used by the dilated
// path (segments of one branch); it is 1 for a plain segment call.
struct View {
    const void *ptr;
    int64_t sb, ss, sh, sn;
};

// Forward over (query block, KV segment) pairs.
struct FwdParams {
    View q, k, v, o, lse;
    int B, S, Hq, Hkv;   // batch, segments per batch entry, heads
    int Nq, Nk;          // rows per (b, s, h)
    int delta;           // visibility: key j <= query i + delta (clamped)
    int noncausal;       // 1: every key visible
    float scale;         // softmax scale (natural units)
    int accumulate;      // fused LSE-merge epilogue into fp32 (o, lse)
    int o_f32;           // output element type: 1 fp32, 0 bf16
    // Head-dependent dilation offsets (0: none).  With hs_r = r > 0 the views
    // select every r-th row of a segment of hs_len rows (row stride r times
    // the tensor's), and query head h starts at row h mod r of the segment:
    // its views move by that many tensor rows and hold
    // ceil((hs_len - h mod r) / r) rows; Nq = Nk is the count at offset 0.
    int hs_r = 0, hs_len = 0;
    int grouped = 0;     // work order (work_item): 0 default, else the band
    // Key-range split (kv_chunk 0: none).  With kv_chunk > 0 (a multiple of
    // 256) the launch runs nchunk work items per query tile: the tile's
    // visible keys [0, e) are cut into parts of len = max(kv_chunk, e / nchunk
    // rounded up to 256) keys, item c taking [c len, (c + 1) len); o and lse
    // are fp32 partials, chunk c at o + c o_chunk and lse + c l_chunk
    // elements.  A chunk past the visible range writes nothing.
    int kv_chunk = 0, nchunk = 1;
    int64_t o_chunk = 0, l_chunk = 0;
};

// Merge of the key-range chunks of a split segment forward (FwdParams'
// kv_chunk) into the call's output: per row, the chunks its query tile
// computed, combined by their log-sum-exp.
struct ChunkMergeParams {
    View o, lse;                 // the call's output
    const float *po, *pl;        // partials: po[c][B][H][N][d], pl[c][B][H][N]
    int B, H, N, d, Nk;
    int delta, noncausal;
    int tile_rows;               // query rows of the forward's work item
    int kv_chunk, nchunk;
    int o_f32;
};

struct MergeParams {
    View oa, la, ob, lb;
    int B, H, N, d;
    int ob_f32;
};

// Backward over (query block, KV segment) pairs; like FwdParams, `S` is an
// extra segment dimension (dilated branches), 1 for a plain segment call.
struct BwdParams {
    View q, k, v, o, lse, dout, dq, dk, dv;
    View dvec;             // D_i = sum_c dO_ic O_ic (fp32), same indexing as lse
    int B, S, Hq, Hkv, Nq, Nk, d;
    int delta, noncausal;
    float scale;
    int o_f32, dk_f32, dv_f32;
    int acc_kv;            // 1: dk, dv (fp32) are accumulated instead of written
    int hs_r = 0, hs_len = 0;  // head-dependent offsets as in FwdParams; query
                           // head h = KV head (one query head per KV head)
    int grouped_kv = 0, grouped_q = 0;  // work order (band) of the dK/dV and dQ launches
};

// Order of a launch's work items, (group, tile) with tile 0 the longest, over
// its workgroups.  The dispatcher hands workgroup i to XCD i mod 8, and each
// XCD has its own L2.  Default order (band 0): the group (batch, segment,
// head) is fastest, so every tile index is spread evenly over the XCDs, which
// suits few groups with many tiles (long causal rows).  Grouped order, for
// many groups with few tiles: XCD x takes groups x, x + 8, ... in bands of
// about `band` tiles (the workgroups an XCD runs at once), longest tile
// first within a band, so a group's tiles run at about the same time and
// read their shared K/V (or Q/dO) rows through one L2, and every XCD takes
// the same tile index at the same slot.  The grouped launch rounds the group
// count up to a multiple of 8; items past the last group are empty.
constexpr int kXcds = 8;
constexpr int kXcdCUs = 32;  // compute units per XCD
struct WorkItem {
    int grp, t;
};
__device__ inline WorkItem work_item(unsigned blk, int ntile, int ngrp, int band)
{
    if (!band)
        return {(int)(blk % (unsigned)ngrp), (int)(blk / (unsigned)ngrp)};
    const int xcd = (int)(blk % kXcds), j = (int)(blk / kXcds);
    const int gx = (ngrp + kXcds - 1) / kXcds;               // groups per XCD
    const int bg = ntile < band ? band / ntile : 1;          // groups per band
    const int bandi = j / (bg * ntile);
    const int nb = min(bg, gx - bandi * bg);                  // groups in this band
    const int idx = j - bandi * bg * ntile;
    return {(bandi * bg + idx % nb) * kXcds + xcd, idx / nb};
}
// A dispatch counts its work-items in 32 bits.
inline bool grid_fits(int64_t blocks, int threads)
{
    return blocks * threads <= (int64_t)0xffffffff;
}
// Band for a launch of ngrp groups of ntile tiles whose XCDs each run `band`
// workgroups at once: grouped when there are groups for every XCD and a
// group's tiles fit in one band, else 0 (default order).
inline int use_grouped(int ntile, int ngrp, int band = kXcdCUs)
{
    return (ngrp >= kXcds && ntile <= band) ? band : 0;
}
inline int64_t work_items(int ntile, int ngrp, int grouped)
{
    const int64_t g = grouped ? ((int64_t)ngrp + kXcds - 1) / kXcds * kXcds : ngrp;
    return g * ntile;
}

// Rows and row shift of head h under head-dependent dilation offsets
// (hs_r > 0); n0 rows and no shift otherwise.
struct HeadRows {
    int n;    // selected rows of this head
    int off;  // offset inside the segment, in tensor rows
};
__host__ __device__ inline HeadRows head_rows(int hs_r, int hs_len, int n0, int h)
{
    if (hs_r <= 0)
        return {n0, 0};
    const int off = h % hs_r;
    const int n = hs_len > off ? (hs_len - off + hs_r - 1) / hs_r : 0;
    return {n, off};
}

// Element shift of a view's first row for offset `off` (its row stride is
// hs_r tensor rows; the kernels address rows with 32-bit strides).
__host__ __device__ inline int64_t head_shift_elems(const View &v, int hs_r, int off)
{
    return hs_r > 0 ? (int64_t)off * ((int)v.sn / hs_r) : 0;
}

// Copy of (flat head f, row n) vectors between two strided layouts; strides
// in bytes, a vector is `units` 16-byte units.  f = b * src_h + h on the
// source side and b * dst_h + h on the destination side.
struct RelayoutParams {
    const char *src;
    char *dst;
    int64_t s_sb, s_sh, s_sn;
    int64_t d_sb, d_sh, d_sn;
    uint32_t src_h, dst_h, F, N, units;
    int head_fast;  // 1: consecutive lanes walk heads of one row, 0: rows of one head
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_fwd_bf16(const FwdParams &p, int d, hipStream_t st);
hipError_t launch_fwd_f32(const FwdParams &p, int d, hipStream_t st);
hipError_t launch_lse_merge(const MergeParams &p, hipStream_t st);
hipError_t launch_chunk_merge(const ChunkMergeParams &p, hipStream_t st);
// Writes the empty partial (O = 0, LSE = -inf) into an fp32/bf16 o view and lse.
hipError_t launch_fill_empty(const View &o, const View &lse, int B, int S, int H,
                             int N, int d, int o_f32, hipStream_t st);
// Casts an fp32 [B][H][N][d] view to a bf16 view.
hipError_t launch_cast_bf16(const View &src, const View &dst, int B, int H, int N,
                            int d, hipStream_t st);
// D = rowsum(dO o O) over p's [B][S][Hq][Nq] rows into p.dvec.
hipError_t launch_bwd_prep(const BwdParams &p, hipStream_t st);
// dK/dV and dQ launches (D must already be in p.dvec).
hipError_t launch_bwd_bf16(const BwdParams &p, hipStream_t st);
// Zero an fp32 [B][H][N][d] view.
hipError_t launch_zero_f32(const View &x, int B, int H, int N, int d, hipStream_t st);
hipError_t launch_head_relayout(const RelayoutParams &p, hipStream_t st);

}  // namespace seqattn
