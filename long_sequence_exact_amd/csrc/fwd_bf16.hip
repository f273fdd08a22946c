// Segment forward, bf16 inputs, MFMA path for gfx950 (CDNA4).
//
// Computes the partial attention of a query block against one KV segment
// ("Ultra-Long Sequence Distributed Transformer", Abstract: each GPU computes
// a partial self-attention for its segment) as (O, LSE), with an optional
// fused log-sum-exp merge into a running fp32 partial, which is what a ring
// step needs ("Boosting Spec Eagle: USP For Long-Context Training", The
// Solution).  The tiled, never-materialised softmax follows the blockwise /
// FlashAttention-style evaluation the pages name as the basis of LongNet's
// kernels ("LongNet ...", Results); the tiling below is designed for gfx950.
//
// Work decomposition
//   * one workgroup = 8 waves = 256 query rows of one (batch, segment, head);
//     each wave owns 32 query rows for the whole kernel; two waves share a
//     SIMD (four at d = 64, two workgroups per CU), so one wave's softmax
//     VALU work can overlap another's MFMAs.  Two other shapes: a long
//     d = 128 call that writes its own output, with enough query tiles for
//     four workgroups per CU, takes 12 waves (384 rows, three per SIMD) with
//     64-key tiles, and a causal d = 64 launch, or one too small to fill
//     the chip, takes 4 waves (128 rows, four workgroups per CU);
//   * the workgroup walks the KV segment in tiles of 128 keys (64 at
//     d = 64), double-buffered in LDS and filled by direct HBM -> LDS buffer
//     loads (rows past the segment end read as zeros), so staging costs no
//     VGPRs and one
//     barrier per tile orders the fill of tile t+1 after every wave's reads
//     of tile t-1; rows are unpadded and XOR-swizzled per 16-byte chunk so
//     the operand reads are bank-conflict free; V stays row-major and is
//     read transposed (ds_read_b64_tr_b16) as the A operand of the PV product;
//   * per tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//     (K from LDS as the A operand, Q held in VGPRs as the B operand), so the
//     accumulator puts one query row in one lane column: the row max needs a
//     single cross-lane step (lane l <-> l^32) and the row sum none until the
//     epilogue;
//   * the reference max of a row is only raised when new scores exceed it by
//     more than 2^8 (a conditional rescale): the exponentials stay <= 256,
//     which fp32 and bf16 hold with full relative precision, and the O
//     rescale is skipped for most tiles; at d = 128 the tile's max is not
//     even taken unless the exponentials against the current reference sum
//     to more than 2^16 in some lane (then the tile is redone);
//   * P^T is rounded to bf16 in registers and is directly the B operand of
//     O^T += V^T P^T; the transposing reads of V deliver keys in the order of
//     the accumulator's row interleave;
//   * causal tiles above the diagonal are never visited; only tiles that
//     straddle it (or the segment tail) are masked;
//   * workgroups are issued longest-first (last query tile first).  With few
//     (batch, segment, head) groups of many query tiles the group index is
//     fastest, so consecutive workgroups -- which the dispatcher spreads
//     round-robin over the 8 XCDs -- stream the same K/V tiles at about the
//     same time; with many groups of at most 32 query tiles each group's
//     tiles run together on one XCD and share its L2 (work_item).
#include "common.h"

namespace seqattn {
namespace {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kWaves = 8;
constexpr int kBQ = 32 * kWaves;      // query rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 headroom before the max is raised
constexpr float kLazyBound = 65536.f;  // largest lane sum of P kept without a rescale (d = 128)
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ inline unsigned pack_bf16(float a, float b)
{
    // two floats -> two bf16, round-to-nearest-even, one v_cvt_pk_bf16_f32
    const f32x2 x = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
}

// Buffer resource over `bytes` bytes at p: loads past the end return zeros,
// which is how rows beyond a segment's end are padded without branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, kRsrcWord3);
}

// The same for a byte count already known to fit in 31 bits (a head's rows
// span less than 2 GiB): the clamp stays in 32-bit scalar arithmetic.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc32(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, max(bytes, 0), kRsrcWord3);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Four bf16 of a transposing LDS read (ds_read_b64_tr_b16): within each group
// of 16 lanes, lane l receives element l%4 of the 8-byte vectors addressed by
// lanes 4e + (l%16)/4, e = 0..3, of its group.
__device__ inline v4i16 read_tr(const bf16 *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)((__attribute__((address_space(3))) char *)(
            (__attribute__((address_space(3))) bf16 *)p)));
}

// The same read at LDS byte offset `off`.
__device__ inline v4i16 read_tr_lds(unsigned off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(uintptr_t)off);
}

// XOR swizzles of the unpadded K and V tiles (16-byte chunk index within a
// row).  K is read as MFMA operands, 16 lanes = 16 consecutive rows x one
// chunk per phase: the swizzle must spread those over all 16 bank groups of
// 16 bytes.  V is read by transposing 8-byte reads, a phase = 4 consecutive
// rows x 4 chunks (64 bytes each): the swizzle must move each row's 4 chunks
// to a different bank group of 64 bytes.
template <int D>
__device__ inline int kswz(int row)
{
    return D == 128 ? (row & 15) : ((row >> 1) & 7);  // 256-byte or 128-byte rows
}
template <int D>
__device__ inline int vswz(int row)
{
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Max and sum of x over lanes l and l ^ 32 (the two halves of a query's
// column in the 32x32 accumulator) without the LDS crossbar: permlane32_swap
// with x in both operands returns, in every lane, x of lane l & 31 and x of
// lane (l & 31) + 32, so both halves form the same value.
__device__ inline float lane_pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float lane_pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// BK keys per K/V tile, NW waves (32 query rows each) per workgroup.  Shapes
// launched: d = 128 with 128-key tiles, 8 waves, two per SIMD; d = 128 with
// 64-key tiles, 12 waves, three per SIMD (168 VGPRs); d = 64 with 64-key
// tiles (at most 128 VGPRs, 32 KiB of LDS), four waves per SIMD: two 8-wave
// or four 4-wave workgroups per CU.
template <int D, int BK, int NW = kWaves, bool SPLIT = false>
__global__ __launch_bounds__(64 * NW, D == 64 ? 4 : (BK == 64 ? 3 : 2)) void fwd_bf16_kernel(const FwdParams p)
{
    constexpr int kBQ = 32 * NW;
    constexpr int ROWB = D * 2;                  // unpadded row of D/8 16-byte chunks
    constexpr int NCH = D / 8;
    constexpr int RPP = 1024 / ROWB;             // rows per 1 KiB DMA piece
    constexpr int TILEB = BK * ROWB;             // bytes per K or V tile
    constexpr int NPC = TILEB / 1024;            // DMA pieces per tile
    constexpr int PPW = (NPC + NW - 1) / NW;     // DMA pieces per wave (at most)
    __shared__ __attribute__((aligned(1024))) char lds[2 * 2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int l32 = lane & 31, hl = lane >> 5;

    const int nqt = (p.Nq + kBQ - 1) / kBQ;
    const int BH = p.B * p.S * p.Hq;
    // a split launch runs nchunk items per query tile, chunk index fastest
    const int chunk = SPLIT ? (int)(blockIdx.x % (unsigned)p.nchunk) : 0;
    const unsigned item = SPLIT ? blockIdx.x / (unsigned)p.nchunk : blockIdx.x;
    const WorkItem wi = work_item(item, nqt, BH, p.grouped);
    if (wi.grp >= BH)
        return;  // padding item of a grouped launch
    const int qt = nqt - 1 - wi.t;
    const int bh = wi.grp;
    const int h = bh % p.Hq;
    const int bs = bh / p.Hq;
    const int s = bs % p.S, b = bs / p.S;
    const int g = (int)(((int64_t)h * p.Hkv) / p.Hq);
    // rows of this head (fewer, and shifted, under head-dependent offsets)
    const HeadRows hr = head_rows(p.hs_r, p.hs_len, p.Nq, h);
    const int Nq = hr.n, Nk = p.hs_r > 0 ? hr.n : p.Nk;
    const int q0 = qt * kBQ;
    if (q0 >= Nq)
        return;  // past this head's rows
    const int64_t rq = head_shift_elems(p.q, p.hs_r, hr.off);
    const int64_t rk = head_shift_elems(p.k, p.hs_r, hr.off);
    const int64_t rv = head_shift_elems(p.v, p.hs_r, hr.off);

    const bf16 *Q = (const bf16 *)p.q.ptr + b * p.q.sb + s * p.q.ss + h * p.q.sh + rq;
    const bf16 *K = (const bf16 *)p.k.ptr + b * p.k.sb + s * p.k.ss + g * p.k.sh + rk;
    const bf16 *V = (const bf16 *)p.v.ptr + b * p.v.sb + s * p.v.ss + g * p.v.sh + rv;
    // valid bytes of each view: rows past Nq / Nk read as zeros
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q, ((int64_t)(Nq - 1) * p.q.sn + D) * 2);

    const int q0w = q0 + wave * 32;
    const int qrow = q0w + l32;

    int kv_end = Nk;
    if (!p.noncausal) {
        const int lim = q0 + kBQ + p.delta;  // keys < lim can be visible
        kv_end = min(kv_end, max(lim, 0));
    }
    int t_begin = 0;  // first key tile (even: the buffers alternate from it)
    if constexpr (SPLIT) {
        // this tile's visible keys in nchunk equal parts (whole 256-key
        // steps, at least kv_chunk keys), so a causal launch's items shrink
        // with their tiles and heavy-first dispatch pairs long with short
        const int len = max(p.kv_chunk, ((kv_end + p.nchunk - 1) / p.nchunk + 255) / 256 * 256);
        const int jb = chunk * len;
        if (jb >= kv_end)
            return;  // nothing of this chunk is visible: the merge skips it
        kv_end = min(kv_end, jb + len);
        t_begin = jb / BK;
    }
    const int ntiles = (kv_end + BK - 1) / BK;

    if (ntiles == 0 && p.accumulate)
        return;  // empty partial: the running accumulator is unchanged

    // Q tile as the B operand of S^T = K Q^T: lane (l32, hl) holds row qrow,
    // d = 16*kk + 8*hl .. +8 (rows past Nq read as zeros).
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = __builtin_bit_cast(bf16x8, load16(qr, (qrow * (int)p.q.sn + kk * 16 + hl * 8) * 2));

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oacc[i][e] = 0.f;

    float m_run = -INFINITY;  // running reference max, in units of log2
    float l_run = 0.f;        // this lane's partial row sum
    bool all_ref = false;     // every row of the wave has a finite reference
    const float c = p.scale * kLog2e;

    // K/V tiles go HBM -> LDS by direct buffer loads into unpadded rows, in
    // 1 KiB pieces: this wave loads pieces wave + NW u (u = 0, 1, ...), piece
    // i covering tile rows RPP i .. +RPP; lane L fills LDS chunk L of the
    // piece = row RPP i + L/NCH, physical chunk L%NCH, which holds logical
    // chunk (L%NCH) ^ swizzle(row) (kswz, vswz).  Piece wave + NW u lies
    // RPP NW u rows below piece `wave`, a multiple of both swizzles' period
    // (16 rows), so all of a wave's pieces share one lane offset and differ
    // by a scalar offset.  The lane offsets are also the same for every
    // tile; each tile moves the buffer resources' base and size instead
    // (scalar work), so rows past the segment end still read as zeros.
    static_assert(PPW == 1 || (RPP * NW) % 16 == 0, "pieces of a wave share the swizzle");
    int koff, voff;
    {
        const int row = RPP * wave + lane / NCH;
        const int ph = lane % NCH;
        koff = (row * (int)p.k.sn + ((ph ^ kswz<D>(row)) * 8)) * 2;
        voff = (row * (int)p.v.sn + ((ph ^ vswz<D>(row)) * 8)) * 2;
    }
    const int kbytes = Nk > 0 ? (int)(((int64_t)(Nk - 1) * p.k.sn + D) * 2) : 0;
    const int vbytes = Nk > 0 ? (int)(((int64_t)(Nk - 1) * p.v.sn + D) * 2) : 0;
    auto issue_tile = [&](int t) {
        const int j0 = t * BK;
        char *kb = lds + (t & 1) * TILEB;          // K buffers, then V buffers
        char *vb = kb + 2 * TILEB;
        const int ks = j0 * (int)p.k.sn * 2, vs = j0 * (int)p.v.sn * 2;
        const __amdgpu_buffer_rsrc_t kt = make_rsrc32((const char *)K + ks, kbytes - ks);
        const __amdgpu_buffer_rsrc_t vt = make_rsrc32((const char *)V + vs, vbytes - vs);
#pragma unroll
        for (int u = 0; u < PPW; ++u) {
            const int piece = wave + NW * u;
            if (NPC % NW != 0 && piece >= NPC)
                break;
            const int ko = koff, vo = voff;
            const int ksu = u * RPP * NW * (int)p.k.sn * 2, vsu = u * RPP * NW * (int)p.v.sn * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kt, (__attribute__((address_space(3))) void *)(kb + piece * 1024), 16, ko, ksu, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vt, (__attribute__((address_space(3))) void *)(vb + piece * 1024), 16, vo, vsu, 0, 0);
        }
    };

    // LDS read offsets: K operand (row 32 kb + l32, logical chunk 2 kk + hl);
    // V^T operand (row 16 ks + 8 rr + 4 (gg/2) + ip/4, logical chunk
    // 4 i + 2 (gg%2) + (ip%4)/2, 8-byte half ip%2)
    const int ksw = kswz<D>(l32);  // rows 32 kb + l32 share l32's swizzle
    const int gg = lane >> 4, ip = lane & 15;
    const int vrow = 4 * (gg >> 1) + (ip >> 2);  // + 16 ks + 8 rr, same swizzle
    const int vbase = vrow * ROWB + (2 * (gg & 1) + ((ip & 3) >> 1)) * 16 + (ip & 1) * 8;
    const int vsw = vswz<D>(vrow) >> 2;
    unsigned vlane[D / 32];  // lane offset of each 32-column block of V^T
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
        vlane[i] = vbase + ((i ^ vsw) << 6);

    if (ntiles > t_begin)
        issue_tile(t_begin);

    // one tile; kbuf and vbuf are the tile's K and V buffers (the loop below
    // runs two tiles per iteration, so both are known addresses and the LDS
    // reads take them as immediate offsets)
    auto step = [&](int t, const char *kbuf, const char *vbuf) {
        // tile t landed (own loads, then everyone's) and every wave is done
        // with tile t-1, whose buffer tile t+1 now fills
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < ntiles)
            issue_tile(t + 1);

        const int j0 = t * BK;
        // whole tile in this wave's causal future: nothing to compute
        if (!p.noncausal && j0 > q0w + 31 + p.delta)
            return;

        f32x16 sacc[BK / 32];
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const bf16x8 a = *(const bf16x8 *)(kbuf + (kb * 32 + l32) * ROWB + (((2 * kk + hl) ^ ksw) * 16));
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kb], 0, 0, 0);
            }
        }
        // keep four K operand reads in flight ahead of the MFMA that uses them
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
        for (int i = 0; i < (BK / 32) * (D / 16) - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

        // accumulator element e of block kb: key j0 + 32kb + 8(e/4) + 4hl + e%4,
        // query qrow
        const bool need_mask = (j0 + BK > Nk) ||
                               (!p.noncausal && j0 + BK - 1 > q0w + p.delta);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = j0 + kb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                    const bool vis = key < Nk && (p.noncausal || key - qrow <= p.delta);
                    if (!vis)
                        sacc[kb][e] = -INFINITY;
                }
        }

        unsigned pk[BK / 32][8];  // P, bf16 pairs
        if constexpr (D == 128) {
            // P = exp2(S c - m) rounded to bf16, and this lane's sum of P
            auto exps = [&](float m) {
                float s0, s1;
#pragma unroll
                for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; e += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], c, -m));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e + 1], c, -m));
                        pk[kb][e >> 1] = pack_bf16(p0, p1);
                        s0 = (kb | e) ? s0 + p0 : p0;  // the first pair starts the sums
                        s1 = (kb | e) ? s1 + p1 : p1;
                    }
                return s0 + s1;
            };

            // Lazy reference: once every row of the wave has one, exponentiate
            // against it without taking the tile's max.  The max and the
            // conditional rescale are taken (and P formed again) only on a
            // row's first keys and when some lane's sum of P exceeds 2^16,
            // so every P kept stays below 2^16 (exact in fp32 and bf16)
            float lsum = 0.f, alpha = 1.f;
            bool redo = !all_ref;
            if (!redo) {
                lsum = exps(m_run);
                redo = __any(!(lsum <= kLazyBound));
            }
            if (redo) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        mx = fmaxf(mx, sacc[kb][e]);
                mx = lane_pair_max(mx);
                const float mxc = mx * c;
                const bool upd = mxc > m_run + kRescaleSlack;
                if (__any(upd)) {
                    const float m_new = upd ? mxc : m_run;
                    alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                    m_run = m_new;
#pragma unroll
                    for (int i = 0; i < D / 32; ++i)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            oacc[i][e] *= alpha;
                }
                lsum = exps((m_run == -INFINITY) ? 0.f : m_run);
                all_ref = !__any(m_run == -INFINITY);
            }
            l_run = l_run * alpha + lsum;
        } else {
            // at d = 64 (short dilated segments) the lazy reference's extra
            // first-tile work and registers cost more than it saves
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    mx = fmaxf(mx, sacc[kb][e]);
            mx = lane_pair_max(mx);

            // conditional rescale: raise the reference max only when some score
            // exceeds it by more than the slack (always on a row's first keys)
            const float mxc = mx * c;
            const bool upd = mxc > m_run + kRescaleSlack;
            const bool any_upd = __any(upd);
            float alpha = 1.f;
            if (any_upd) {
                const float m_new = upd ? mxc : m_run;
                // exp2(-inf) = 0 for a row's first visible keys; rows that keep
                // their max (fully masked ones included) keep alpha = 1
                alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                m_run = m_new;
#pragma unroll
                for (int i = 0; i < D / 32; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        oacc[i][e] *= alpha;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

            float lsum;
#pragma unroll
            for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], c, -m_use));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e + 1], c, -m_use));
                    lsum = (kb | e) ? lsum + (p0 + p1) : p0 + p1;
                    pk[kb][e >> 1] = pack_bf16(p0, p1);
                }
            l_run = l_run * alpha + lsum;
        }

        // the V buffer's LDS offset as an opaque value: the compiler then
        // forms one base per column block and folds the key steps into the
        // reads' offsets (a known address makes it rebuild the base per read)
        unsigned vo = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char *)vbuf;
        asm("" : "+s"(vo));
        unsigned vcol[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
            vcol[i] = vo + vlane[i];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kb = ks >> 1, half = ks & 1;
            u32x4 pw = {pk[kb][half * 4 + 0], pk[kb][half * 4 + 1],
                        pk[kb][half * 4 + 2], pk[kb][half * 4 + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const unsigned base = vcol[i] + 16 * ks * ROWB;
                const v4i16 lo = read_tr_lds(base);
                const v4i16 hi = read_tr_lds(base + 8 * ROWB);
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[i], 0, 0, 0);
            }
        }
        if constexpr (D == 128) {
            // keep four MFMAs' transposed V reads (two each) in flight (the
            // compiler's own order keeps about two)
            constexpr int NM = (BK / 16) * (D / 32);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int u = 0; u < NM - 4; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
    };
    for (int t = t_begin; t < ntiles; t += 2) {
        step(t, lds, lds + 2 * TILEB);
        if (t + 1 < ntiles)
            step(t + 1, lds + TILEB, lds + 3 * TILEB);
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l), optional merge ----
    const float l_tot = lane_pair_sum(l_run);
    const bool has = l_tot > 0.f;
    const float inv = has ? 1.f / l_tot : 0.f;
    const float lse_new = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (qrow >= Nq)
        return;

    const int64_t ro = head_shift_elems(p.o, p.hs_r, hr.off);
    const int64_t rl = head_shift_elems(p.lse, p.hs_r, hr.off);
    float *Lp = (float *)p.lse.ptr + b * p.lse.sb + s * p.lse.ss + h * p.lse.sh + rl +
                (int64_t)qrow * p.lse.sn + chunk * p.l_chunk;
    const int64_t orow = b * p.o.sb + s * p.o.ss + h * p.o.sh + ro + (int64_t)qrow * p.o.sn +
                         chunk * p.o_chunk;

    if (!p.accumulate) {
        if (hl == 0)
            *Lp = lse_new;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = i * 32 + gq * 8 + hl * 4;
                const float x0 = oacc[i][gq * 4 + 0] * inv, x1 = oacc[i][gq * 4 + 1] * inv;
                const float x2 = oacc[i][gq * 4 + 2] * inv, x3 = oacc[i][gq * 4 + 3] * inv;
                if (p.o_f32) {
                    float4 w = {x0, x1, x2, x3};
                    *(float4 *)((float *)p.o.ptr + orow + d0) = w;
                } else {
                    uint2 w = {pack_bf16(x0, x1), pack_bf16(x2, x3)};
                    *(uint2 *)((bf16 *)p.o.ptr + orow + d0) = w;
                }
            }
        return;
    }

    // fused merge with the running fp32 partial (o, lse): its LSE and every
    // row chunk are read before anything is written, so the reads' round
    // trips overlap
    float *Op = (float *)p.o.ptr + orow;
    const float la = *Lp;
    float4 old[D / 32][4];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
            old[i][gq] = *(const float4 *)(Op + i * 32 + gq * 8 + hl * 4);
    const float M = fmaxf(la, lse_new);
    if (M == -INFINITY)
        return;  // both empty: stays (0, -inf)
    const float wa = __expf(la - M), wb = __expf(lse_new - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb / tot * inv;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d0 = i * 32 + gq * 8 + hl * 4;
            float4 a = old[i][gq];
            a.x = fa * a.x + fb * oacc[i][gq * 4 + 0];
            a.y = fa * a.y + fb * oacc[i][gq * 4 + 1];
            a.z = fa * a.z + fb * oacc[i][gq * 4 + 2];
            a.w = fa * a.w + fb * oacc[i][gq * 4 + 3];
            *(float4 *)(Op + d0) = a;
        }
    if (hl == 0)
        *Lp = M + __logf(tot);
}


}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p0, int d, hipStream_t st)
{
    FwdParams p = p0;
    const int BH = p.B * p.S * p.Hq;
    int nqt = (p.Nq + kBQ - 1) / kBQ;
    if ((int64_t)nqt * BH == 0)
        return hipSuccess;
    if (p.kv_chunk > 0) {
        // a split call (too few query tiles to fill the chip): 8-wave items,
        // nchunk per query tile, in the default order
        if (d != 128 || p.accumulate || p.hs_r > 0 || p.kv_chunk % (2 * 128) != 0)
            return hipErrorInvalidValue;
        p.grouped = 0;
        const int64_t grid = work_items(nqt, BH, 0) * p.nchunk;
        if (!grid_fits(grid, kThreads))
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 128, kWaves, true>), dim3((unsigned)grid), dim3(kThreads), 0, st, p);
        return hipGetLastError();
    }
    const int nqt12 = (p.Nq + 383) / 384;
    if (d == 128 && !p.accumulate && p.Nq >= 16384 &&
        (int64_t)nqt12 * BH >= 4 * kXcds * kXcdCUs) {
        // a long call writing its own output (the Ulysses share at 128K
        // tokens): 12-wave workgroups of 384 rows, three waves per SIMD,
        // measured 1-2% faster there.  It needs at least four workgroups per
        // CU: with fewer, the causal call's longest workgroups set its time
        // and the 8-wave kernel's finer tiles finish sooner (64K tokens, 4
        // heads: 3.63 against 3.76 ms).  The accumulating sweeps (ring and
        // USP steps) and short blocks keep 8 waves (384 does not divide
        // their 2048-row blocks)
        nqt = nqt12;
        p.grouped = use_grouped(nqt, BH, kXcdCUs);
        const int64_t grid = work_items(nqt, BH, p.grouped);
        if (!grid_fits(grid, 768))
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 64, 12>), dim3((unsigned)grid), dim3(768), 0, st, p);
        return hipGetLastError();
    }
    if (d == 128) {
        p.grouped = use_grouped(nqt, BH, kXcdCUs);
        const int64_t grid = work_items(nqt, BH, p.grouped);
        if (!grid_fits(grid, kThreads))
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 128>), dim3((unsigned)grid), dim3(kThreads), 0, st, p);
        return hipGetLastError();
    }
    // d = 64 launches (LongNet's branches) take 64-key tiles at four waves
    // per SIMD: two 8-wave workgroups per CU, so an XCD runs twice as many
    // at once.  A causal launch, or one with fewer workgroups than the chip
    // holds (a long-segment branch selects few rows), takes 4-wave
    // workgroups of 128 rows instead, four per CU: their rows spread over
    // twice as many CUs, and the causal triangle is cut into finer tiles
    // (LongNet's causal page mixture 0.436 against 0.450 ms; the non-causal
    // 32K mixture keeps the 8-wave tiles, 0.622 against 0.627)
    const bool small = (int64_t)nqt * BH < 2 * 256 || !p.noncausal;
    if (small) {
        nqt = (p.Nq + 127) / 128;
        p.grouped = use_grouped(nqt, BH, 4 * kXcdCUs);
        const int64_t grid = work_items(nqt, BH, p.grouped);
        if (!grid_fits(grid, 256))
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 4>), dim3((unsigned)grid), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    p.grouped = use_grouped(nqt, BH, 2 * kXcdCUs);
    const int64_t grid = work_items(nqt, BH, p.grouped);
    if (!grid_fits(grid, kThreads))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_bf16_kernel<64, 64>), dim3((unsigned)grid), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace seqattn
