// Segment backward, bf16 inputs, MFMA path for gfx950.
//
// Gradients of one (query block, KV segment) pair given the GLOBAL softmax
// statistics (LSE and O merged over every segment the queries saw): a device
// that attended to a segment forms the gradients for that segment's keys and
// values ("LongNet: Scaling Transformers to 1,000,000,000 Tokens",
// Distributed Trainer: the backward turns the all-gather into a
// reduce-scatter).  With P = exp(sigma*S - LSE) and D_i = dO_i . O_i:
//   dV = P^T dO,  dS = P o (dO V^T - D),  dK = sigma dS^T Q,  dQ += sigma dS K.
//
// Work decomposition (three launches at d = 128; at d = 64 the dK/dV and dQ
// items share one launch, bwd_kvdq)
//   * bwd_prep: D_i for every query row (HBM-bound, 16 lanes per row, rows
//     strided over a capped grid);
//   * bwd_main (dK, dV, d = 128): one workgroup = 8 waves for 128 keys of one
//     (batch, KV head): waves 0-3 accumulate dV^T and waves 4-7 dK^T for the
//     same 4 x 32 keys (one fp32 accumulator per wave keeps two waves per
//     SIMD), looping over the query heads sharing the KV head and over the
//     visible 64-row query tiles.  Per tile the dV wave recomputes
//     S = Q K^T with keys in lane columns (v_mfma_f32_32x32x16_bf16) and
//     P, so P is directly the B operand of dV^T += dO^T P, and hands P
//     (bf16) through LDS to the dK wave of its pair, which takes the tile
//     one step later: dP = dO V^T, dS = P o (dP - D), dK^T += Q^T dS.  The
//     lag lets one barrier per step order both the hand-over and the Q / dO
//     tiles, which sit in three LDS buffers (the dV waves' tile, the dK
//     waves' tile and the next one, stored from VGPRs loaded a step ahead
//     with range-checked buffer loads).  The Q^T and dO^T A operands are
//     read from the row-major tiles with transposing reads
//     (ds_read_b64_tr_b16);
//   * bwd_kv (dK, dV, d = 64): the same with 8 x 32 keys per workgroup and
//     both accumulators in each wave, which fit at d = 64, so S and P are
//     formed once per pair;
//   * bwd_dq (dQ): query-tile major, shaped like the forward kernel (below).
//     Recomputing S and dP there costs two more contractions than sharing
//     them with bwd_main, but dQ then needs no atomics and no round trip of
//     dS through LDS, and the result is deterministic.
#include "common.h"

namespace seqattn {
namespace {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 128;          // keys per workgroup (32 per wave pair)
constexpr int kBQ = 64;            // query rows per iteration
constexpr float kLog2e = 1.4426950408889634f;
// MFMAs' worth of LDS operand reads kept in flight in the d = 64 blocks (the
// d = 128 kernels keep four: six measured no faster there, and slower in the
// dK/dV kernel)
constexpr int AHEAD = 6;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ inline unsigned pack_bf16(float a, float b)
{
    // two floats -> two bf16, round-to-nearest-even, one v_cvt_pk_bf16_f32
    const f32x2 x = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
}

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// D_i = sum_c dO_ic O_ic; 16 lanes per row, d/16 elements per lane, rows
// strided over the grid.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p)
{
    const int64_t rows = (int64_t)p.B * p.S * p.Hq * p.Nq;
    const int64_t step = (int64_t)gridDim.x * (256 / 16);
    const int sub = threadIdx.x & 15;
    const int per = p.d / 16;  // 4 or 8
    // every lane of a 16-lane group runs the same rows, so the shuffle below
    // always has all 16 partners
    for (int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16; row < rows; row += step) {
        const int i = (int)(row % p.Nq);
        int64_t r = row / p.Nq;
        const int h = (int)(r % p.Hq);
        r /= p.Hq;
        const int s = (int)(r % p.S);
        const int b = (int)(r / p.S);
        const bf16 *dO = (const bf16 *)p.dout.ptr + b * p.dout.sb + s * p.dout.ss +
                         h * p.dout.sh + (int64_t)i * p.dout.sn + sub * per;
        const int64_t ooff = b * p.o.sb + s * p.o.ss + h * p.o.sh + (int64_t)i * p.o.sn + sub * per;
        float acc = 0.f;
        for (int c = 0; c < per; c += 4) {
            const uint2 g = *(const uint2 *)(dO + c);
            float o0, o1, o2, o3;
            if (p.o_f32) {
                const float4 x = *(const float4 *)((const float *)p.o.ptr + ooff + c);
                o0 = x.x; o1 = x.y; o2 = x.z; o3 = x.w;
            } else {
                const uint2 x = *(const uint2 *)((const bf16 *)p.o.ptr + ooff + c);
                o0 = bf16_lo(x.x); o1 = bf16_hi(x.x); o2 = bf16_lo(x.y); o3 = bf16_hi(x.y);
            }
            acc += bf16_lo(g.x) * o0 + bf16_hi(g.x) * o1 + bf16_lo(g.y) * o2 + bf16_hi(g.y) * o3;
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1)
            acc += __shfl_xor(acc, m, 16);
        if (sub == 0)
            *((float *)p.dvec.ptr + b * p.dvec.sb + s * p.dvec.ss + h * p.dvec.sh +
              (int64_t)i * p.dvec.sn) = acc;
    }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(View x, int B, int H, int N, int d)
{
    const int tpr = d / 4;
    const int64_t total = (int64_t)B * H * N * tpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += stride) {
        const int64_t row = gid / tpr;
        const int c4 = (int)(gid % tpr) * 4;
        const int n = (int)(row % N);
        const int64_t bh = row / N;
        const int h = (int)(bh % H), b = (int)(bh / H);
        *(float4 *)((float *)x.ptr + b * x.sb + h * x.sh + (int64_t)n * x.sn + c4) =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int D>
struct BCfg {
    static constexpr int BQ = kBQ;  // query rows per iteration
    static constexpr int CPT = BQ * D / 8 / kThreads;  // 16-byte chunks per thread per tile
    static_assert(CPT * kThreads * 8 == BQ * D, "tile split");
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, kRsrcWord3);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ds_read_b64_tr_b16: within each 16-lane group, lane l receives element l%4
// of the 8-byte vectors addressed by lanes 4e + (l%16)/4, e = 0..3.
__device__ inline v4i16 read_tr(const bf16 *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)((__attribute__((address_space(3))) char *)(
            (__attribute__((address_space(3))) bf16 *)p)));
}

__device__ inline bf16x8 cat_tr(v4i16 lo, v4i16 hi)
{
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The Q / dO tiles (dK/dV kernel) and the K tile (dQ kernel) are read two
// ways: as MFMA row operands (a read phase = 16 consecutive rows x one
// 16-byte chunk) and by transposing reads (a phase = 4 consecutive rows x 4
// chunks).  Rows are unpadded (D/8 chunks of 16 bytes); logical chunk c of
// row r sits at c ^ tswz(r).  The swizzle is a bijection on the 16 (d = 128)
// or, per row parity, 8 (d = 64) rows of a phase of the first kind and puts
// each of 4 consecutive rows in a different 64-byte bank group, so neither
// kind of read conflicts.
template <int D>
__device__ inline int tswz(int row)
{
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                    : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// byte offset of logical chunk c of row r in a swizzled tile
template <int D>
__device__ inline int swz_off(int r, int c)
{
    return r * (2 * D) + ((c ^ tswz<D>(r)) << 4);
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(const BwdParams p)
{
    using C = BCfg<D>;
    constexpr int BQ = C::BQ;
    constexpr int TB = BQ * 2 * D;           // bytes of one Q or dO tile
    constexpr int PB = (BQ / 32) * 64 * 32;  // bytes of one wave pair's P tile
    // Q / dO tiles in three buffers: the dV waves read tile it, the dK waves
    // tile it - 1, and tile it + 1 is stored meanwhile
    __shared__ __attribute__((aligned(16))) char Qs[3 * TB];
    __shared__ __attribute__((aligned(16))) char dOs[3 * TB];
    // P of each wave pair, written by its dV wave, read one step later by
    // its dK wave (double-buffered), in the accumulator's lane layout (per
    // 32-query block: lane l's first 16 bytes at 16 l, its last 16 at 1024 + 16 l)
    __shared__ __attribute__((aligned(16))) char Ps[2 * 4 * PB];
    __shared__ float lse2s[3][BQ];
    __shared__ float Dsh[3][BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_dk = wave >= 4;
    const int pair = wave & 3;
    const int l32 = lane & 31, hl = lane >> 5;
    const int gg = lane >> 4, ip = lane & 15;

    const int nkt = (p.Nk + kBKV - 1) / kBKV;
    const WorkItem wi = work_item(blockIdx.x, nkt, p.B * p.S * p.Hkv, p.grouped_kv);
    if (wi.grp >= p.B * p.S * p.Hkv)
        return;  // padding item of a grouped launch
    const int kt = wi.t;  // first key tiles see the most query rows
    const int bsg = wi.grp;
    const int g = bsg % p.Hkv, bs = bsg / p.Hkv;
    const int s = bs % p.S, b = bs / p.S;
    const int k0 = kt * kBKV;
    const int kw0 = k0 + pair * 32;
    const int key = kw0 + l32;  // this lane's key (accumulator column)
    const HeadRows hr = head_rows(p.hs_r, p.hs_len, p.Nk, g);
    const int Nk = hr.n, Nq = p.hs_r > 0 ? hr.n : p.Nq;
    if (k0 >= Nk)
        return;  // past this head's rows

    const bf16 *K = (const bf16 *)p.k.ptr + b * p.k.sb + s * p.k.ss + g * p.k.sh +
                    head_shift_elems(p.k, p.hs_r, hr.off);
    const bf16 *V = (const bf16 *)p.v.ptr + b * p.v.sb + s * p.v.ss + g * p.v.sh +
                    head_shift_elems(p.v, p.hs_r, hr.off);
    const int64_t sq = head_shift_elems(p.q, p.hs_r, hr.off);
    const int64_t so = head_shift_elems(p.dout, p.hs_r, hr.off);
    const int64_t sl = head_shift_elems(p.lse, p.hs_r, hr.off);
    const int64_t sd = head_shift_elems(p.dvec, p.hs_r, hr.off);

    // B operands (k = d): K rows for the dV waves' S, V rows for the dK
    // waves' dP; lane holds key `key`, d = 16kk + 8hl .. +8
    bf16x8 rB[D / 16];
    {
        const bf16 *R = is_dk ? V : K;
        const int64_t rs = is_dk ? p.v.sn : p.k.sn;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (key < Nk)
                x = *(const u32x4 *)(R + (int64_t)key * rs + kk * 16 + hl * 8);
            rB[kk] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 acc[D / 32];  // dV^T (waves 0-3) or dK^T / sigma (waves 4-7)
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[i][e] = 0.f;

    const float c = p.scale * kLog2e;
    const int group = p.Hq / p.Hkv;
    const int nqt = (Nq + BQ - 1) / BQ;
    int qt_begin = 0;
    if (!p.noncausal) {
        const int first_q = max(0, k0 - p.delta);  // smallest query seeing key k0
        qt_begin = min(nqt, first_q / BQ);
    }
    const int per_head = nqt - qt_begin;
    const int niters = group * per_head;

    u32x4 qreg[C::CPT], oreg[C::CPT];
    float lreg = 0.f, dreg = 0.f;
    int srow[C::CPT], scol[C::CPT];
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
        const int ch = tid + u * kThreads;
        srow[u] = ch / (D / 8);
        scol[u] = (ch % (D / 8)) * 8;
    }
    auto prefetch = [&](int it) {
        const int h = g * group + it / per_head;
        const int q0 = (qt_begin + it % per_head) * BQ;
        const bf16 *Q = (const bf16 *)p.q.ptr + b * p.q.sb + s * p.q.ss + h * p.q.sh + sq;
        const bf16 *dO = (const bf16 *)p.dout.ptr + b * p.dout.sb + s * p.dout.ss +
                         h * p.dout.sh + so;
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q, ((int64_t)(Nq - 1) * p.q.sn + D) * 2);
        const __amdgpu_buffer_rsrc_t orr = make_rsrc(dO, ((int64_t)(Nq - 1) * p.dout.sn + D) * 2);
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            qreg[u] = load16(qr, ((q0 + srow[u]) * (int)p.q.sn + scol[u]) * 2);
            oreg[u] = load16(orr, ((q0 + srow[u]) * (int)p.dout.sn + scol[u]) * 2);
        }
        if (tid < BQ) {
            const int i = q0 + tid;
            // raw values: the stage formats them a step later, so no wait
            // for these loads (or the tile loads before them) falls here
            lreg = -INFINITY;  // a row past the end contributes P = 0
            dreg = 0.f;
            if (i < Nq) {
                lreg = *((const float *)p.lse.ptr + b * p.lse.sb + s * p.lse.ss +
                         h * p.lse.sh + sl + (int64_t)i * p.lse.sn);
                dreg = *((const float *)p.dvec.ptr + b * p.dvec.sb + s * p.dvec.ss +
                         h * p.dvec.sh + sd + (int64_t)i * p.dvec.sn);
            }
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            *(u32x4 *)(Qs + buf * TB + swz_off<D>(srow[u], scol[u] >> 3)) = qreg[u];
            *(u32x4 *)(dOs + buf * TB + swz_off<D>(srow[u], scol[u] >> 3)) = oreg[u];
        }
        if (tid < BQ) {
            // LSE in log2 units; -inf (no visible key) becomes +inf: P = 0
            lse2s[buf][tid] = lreg == -INFINITY ? INFINITY : lreg * kLog2e;
            Dsh[buf][tid] = -dreg;  // -D: the dP accumulators start from it
        }
    };

    const int trow = 4 * (gg >> 1) + (ip >> 2);

    if (niters > 0) {
        prefetch(0);
        stage(0);
        if (niters > 1)
            prefetch(1);
    }

    // step it: the dV waves take tile it, the dK waves tile it - 1
    for (int it = 0; it <= niters && niters > 0; ++it) {
        // tile it staged, P(it - 1) written, and buffer (it + 1) % 3 (tile
        // it - 2) no longer read
        __syncthreads();
        if (it + 1 < niters) {
            stage((it + 1) % 3);
            if (it + 2 < niters)
                prefetch(it + 2);
        }
        const int tq = is_dk ? it - 1 : it;  // this wave's tile
        if (tq < 0 || tq >= niters)
            continue;
        const int buf = tq % 3;
        const char *Qb = Qs + buf * TB;
        const char *Ob = dOs + buf * TB;
        char *Pp = Ps + ((tq & 1) * 4 + pair) * PB + lane * 16;
        const int q0 = (qt_begin + tq % per_head) * BQ;

        unsigned pB[BQ / 32][8];  // P (dV waves) or dS (dK waves), bf16 pairs
        if (!is_dk) {
            const bool need_mask = (kw0 + 32 > Nk) || (q0 + BQ > Nq) ||
                                   (!p.noncausal && kw0 + 31 > q0 + p.delta);
#pragma unroll
            for (int qb = 0; qb < BQ / 32; ++qb) {
                f32x16 sv;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    sv[e] = 0.f;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8 aq = *(const bf16x8 *)(Qb + swz_off<D>(qb * 32 + l32, 2 * kk + hl));
                    sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, rB[kk], sv, 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int u = 0; u < D / 16 - 4; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                // masked scores become -inf (P = 0) before the exponentials,
                // which then run unconditionally
                if (need_mask) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int qi = q0 + qb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                        const bool vis = (key < Nk) & (qi < Nq) &
                                         (p.noncausal | (key - qi <= p.delta));
                        sv[e] = vis ? sv[e] : -INFINITY;
                    }
                }
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int r0 = qb * 32 + gq * 8 + hl * 4;
                    const float4 l2 = *(const float4 *)(&lse2s[buf][r0]);
                    const float lv[4] = {l2.x, l2.y, l2.z, l2.w};
                    float pv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        pv[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[gq * 4 + u], c, -lv[u]));
                    pB[qb][gq * 2 + 0] = pack_bf16(pv[0], pv[1]);
                    pB[qb][gq * 2 + 1] = pack_bf16(pv[2], pv[3]);
                }
                // hand P to the dK wave of the pair (read next step)
                *(u32x4 *)(Pp + qb * 2048) = u32x4{pB[qb][0], pB[qb][1], pB[qb][2], pB[qb][3]};
                *(u32x4 *)(Pp + qb * 2048 + 1024) = u32x4{pB[qb][4], pB[qb][5], pB[qb][6], pB[qb][7]};
            }
        } else {
#pragma unroll
            for (int qb = 0; qb < BQ / 32; ++qb) {
                // dP - D: the accumulator starts at -D of its query rows
                f32x16 dp;
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const float4 nd = *(const float4 *)(&Dsh[buf][qb * 32 + gq * 8 + hl * 4]);
                    dp[gq * 4 + 0] = nd.x;
                    dp[gq * 4 + 1] = nd.y;
                    dp[gq * 4 + 2] = nd.z;
                    dp[gq * 4 + 3] = nd.w;
                }
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8 ad = *(const bf16x8 *)(Ob + swz_off<D>(qb * 32 + l32, 2 * kk + hl));
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, rB[kk], dp, 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int u = 0; u < D / 16 - 4; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                // P from the dV wave (zero where masked), dS = P o (dP - D)
                const u32x4 w0 = *(const u32x4 *)(Pp + qb * 2048);
                const u32x4 w1 = *(const u32x4 *)(Pp + qb * 2048 + 1024);
                const unsigned pw[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const unsigned a0 = pw[gq * 2 + 0], a1 = pw[gq * 2 + 1];
                    const float d0 = bf16_lo(a0) * dp[gq * 4 + 0];
                    const float d1 = bf16_hi(a0) * dp[gq * 4 + 1];
                    const float d2 = bf16_lo(a1) * dp[gq * 4 + 2];
                    const float d3 = bf16_hi(a1) * dp[gq * 4 + 3];
                    pB[qb][gq * 2 + 0] = pack_bf16(d0, d1);
                    pB[qb][gq * 2 + 1] = pack_bf16(d2, d3);
                }
            }
        }

        // ---- dV^T += dO^T P or dK^T += Q^T dS (k = the tile's BQ query rows) ----
        const char *At = is_dk ? Qb : Ob;
#pragma unroll
        for (int ks = 0; ks < BQ / 16; ++ks) {
            const int qb = ks >> 1, half = ks & 1;
            u32x4 w = {pB[qb][half * 4 + 0], pB[qb][half * 4 + 1], pB[qb][half * 4 + 2],
                       pB[qb][half * 4 + 3]};
            const bf16x8 bb = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const int cc = 4 * i + 2 * (gg & 1) + ((ip & 3) >> 1);
                const int o0 = swz_off<D>(16 * ks + trow, cc) + (ip & 1) * 8;
                const int o1 = swz_off<D>(16 * ks + 8 + trow, cc) + (ip & 1) * 8;
                const bf16x8 a = cat_tr(read_tr((const bf16 *)(At + o0)), read_tr((const bf16 *)(At + o1)));
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[i], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int u = 0; u < (BQ / 16) * (D / 32) - 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }

    // ---- write dK = sigma (dK^T)^T or dV (key rows, 4 consecutive d per store) ----
    if (key >= Nk)
        return;
    const View &out = is_dk ? p.dk : p.dv;
    const int out_f32 = is_dk ? p.dk_f32 : p.dv_f32;
    const float f = is_dk ? p.scale : 1.f;
    const int64_t krow = b * out.sb + s * out.ss + g * out.sh +
                         head_shift_elems(out, p.hs_r, hr.off) + (int64_t)key * out.sn;
    // accumulated output: every running sum read before any is written
    float4 old[D / 32][4];
    if (p.acc_kv) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                old[i][gq] = *(const float4 *)((const float *)out.ptr + krow + i * 32 + gq * 8 + hl * 4);
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d0 = i * 32 + gq * 8 + hl * 4;
            const float x0 = acc[i][gq * 4 + 0] * f, x1 = acc[i][gq * 4 + 1] * f;
            const float x2 = acc[i][gq * 4 + 2] * f, x3 = acc[i][gq * 4 + 3] * f;
            if (p.acc_kv) {  // fp32, accumulated
                float4 w = old[i][gq];
                w.x += x0; w.y += x1; w.z += x2; w.w += x3;
                *(float4 *)((float *)out.ptr + krow + d0) = w;
            } else if (out_f32) {
                float4 w = {x0, x1, x2, x3};
                *(float4 *)((float *)out.ptr + krow + d0) = w;
            } else {
                uint2 w = {pack_bf16(x0, x1), pack_bf16(x2, x3)};
                *(uint2 *)((bf16 *)out.ptr + krow + d0) = w;
            }
        }
}

// ---------------------------------------------------------------------------
// dK and dV at d = 64 in one wave: one workgroup = 8 waves = 256 keys of one
// (batch, KV head), wave = 32 keys holding both accumulators (dV^T and
// dK^T / sigma, 2 x 32 VGPRs at d = 64), so S and P are formed once per
// (query, key) pair instead of once per wave of a dV/dK pair.  Staging and
// operand layouts as in bwd_main_kernel.
// ---------------------------------------------------------------------------

template <int D, int BQ, int NW>
__device__ __forceinline__ void bwd_kv_body(const BwdParams &p, unsigned blk)
{
    constexpr int kThreads = 64 * NW, kFKeys = 32 * NW;
    constexpr int CPT = BQ * D / 8 / kThreads;
    static_assert(CPT * kThreads * 8 == BQ * D, "tile split");
    __shared__ __attribute__((aligned(16))) char Qs[BQ * 2 * D];
    __shared__ __attribute__((aligned(16))) char dOs[BQ * 2 * D];
    __shared__ float lse2s[BQ];
    __shared__ float Dsh[BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;
    const int gg = lane >> 4, ip = lane & 15;

    const int nkt = (p.Nk + kFKeys - 1) / kFKeys;
    const WorkItem wi = work_item(blk, nkt, p.B * p.S * p.Hkv, p.grouped_kv);
    if (wi.grp >= p.B * p.S * p.Hkv)
        return;  // padding item of a grouped launch
    const int kt = wi.t;
    const int bsg = wi.grp;
    const int g = bsg % p.Hkv, bs = bsg / p.Hkv;
    const int s = bs % p.S, b = bs / p.S;
    const int k0 = kt * kFKeys;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + l32;
    const HeadRows hr = head_rows(p.hs_r, p.hs_len, p.Nk, g);
    const int Nk = hr.n, Nq = p.hs_r > 0 ? hr.n : p.Nq;
    if (k0 >= Nk)
        return;

    const bf16 *K = (const bf16 *)p.k.ptr + b * p.k.sb + s * p.k.ss + g * p.k.sh +
                    head_shift_elems(p.k, p.hs_r, hr.off);
    const bf16 *V = (const bf16 *)p.v.ptr + b * p.v.sb + s * p.v.ss + g * p.v.sh +
                    head_shift_elems(p.v, p.hs_r, hr.off);
    const int64_t sq = head_shift_elems(p.q, p.hs_r, hr.off);
    const int64_t so = head_shift_elems(p.dout, p.hs_r, hr.off);
    const int64_t sl = head_shift_elems(p.lse, p.hs_r, hr.off);
    const int64_t sd = head_shift_elems(p.dvec, p.hs_r, hr.off);

    bf16x8 kB[D / 16], vB[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
        if (key < Nk) {
            xk = *(const u32x4 *)(K + (int64_t)key * p.k.sn + kk * 16 + hl * 8);
            xv = *(const u32x4 *)(V + (int64_t)key * p.v.sn + kk * 16 + hl * 8);
        }
        kB[kk] = __builtin_bit_cast(bf16x8, xk);
        vB[kk] = __builtin_bit_cast(bf16x8, xv);
    }

    f32x16 accV[D / 32], accK[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            accV[i][e] = accK[i][e] = 0.f;

    const float c = p.scale * kLog2e;
    const int group = p.Hq / p.Hkv;
    const int nqt = (Nq + BQ - 1) / BQ;
    int qt_begin = 0;
    if (!p.noncausal) {
        const int first_q = max(0, k0 - p.delta);
        qt_begin = min(nqt, first_q / BQ);
    }
    const int per_head = nqt - qt_begin;
    const int niters = group * per_head;

    u32x4 qreg[CPT], oreg[CPT];
    float lreg = 0.f, dreg = 0.f;
    int srow[CPT], scol[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = tid + u * kThreads;
        srow[u] = ch / (D / 8);
        scol[u] = (ch % (D / 8)) * 8;
    }
    auto prefetch = [&](int it) {
        const int h = g * group + it / per_head;
        const int q0 = (qt_begin + it % per_head) * BQ;
        const bf16 *Q = (const bf16 *)p.q.ptr + b * p.q.sb + s * p.q.ss + h * p.q.sh + sq;
        const bf16 *dO = (const bf16 *)p.dout.ptr + b * p.dout.sb + s * p.dout.ss +
                         h * p.dout.sh + so;
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q, ((int64_t)(Nq - 1) * p.q.sn + D) * 2);
        const __amdgpu_buffer_rsrc_t orr = make_rsrc(dO, ((int64_t)(Nq - 1) * p.dout.sn + D) * 2);
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            qreg[u] = load16(qr, ((q0 + srow[u]) * (int)p.q.sn + scol[u]) * 2);
            oreg[u] = load16(orr, ((q0 + srow[u]) * (int)p.dout.sn + scol[u]) * 2);
        }
        if (tid < BQ) {
            const int i = q0 + tid;
            // raw values, formatted when staged
            lreg = -INFINITY;
            dreg = 0.f;
            if (i < Nq) {
                lreg = *((const float *)p.lse.ptr + b * p.lse.sb + s * p.lse.ss +
                         h * p.lse.sh + sl + (int64_t)i * p.lse.sn);
                dreg = *((const float *)p.dvec.ptr + b * p.dvec.sb + s * p.dvec.ss +
                         h * p.dvec.sh + sd + (int64_t)i * p.dvec.sn);
            }
        }
    };

    const int trow = 4 * (gg >> 1) + (ip >> 2);

    if (niters > 0)
        prefetch(0);

    for (int it = 0; it < niters; ++it) {
        const int q0 = (qt_begin + it % per_head) * BQ;

        __syncthreads();
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            *(u32x4 *)(Qs + swz_off<D>(srow[u], scol[u] >> 3)) = qreg[u];
            *(u32x4 *)(dOs + swz_off<D>(srow[u], scol[u] >> 3)) = oreg[u];
        }
        if (tid < BQ) {
            lse2s[tid] = lreg == -INFINITY ? INFINITY : lreg * kLog2e;
            Dsh[tid] = -dreg;  // -D: the dP accumulators start from it
        }
        __syncthreads();
        if (it + 1 < niters)
            prefetch(it + 1);

        // this wave's keys all in the future of the whole query tile: nothing
        if (!p.noncausal && kw0 > q0 + BQ - 1 + p.delta)
            continue;
        const bool need_mask = (kw0 + 32 > Nk) || (q0 + BQ > Nq) ||
                               (!p.noncausal && kw0 + 31 > q0 + p.delta);
        unsigned pB[BQ / 32][8], dB[BQ / 32][8];  // P and dS, bf16 pairs
#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb) {
            // dP - D: the dP accumulator starts at -D of its query rows
            f32x16 sv, dp;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const float4 nd = *(const float4 *)(&Dsh[qb * 32 + gq * 8 + hl * 4]);
                dp[gq * 4 + 0] = nd.x;
                dp[gq * 4 + 1] = nd.y;
                dp[gq * 4 + 2] = nd.z;
                dp[gq * 4 + 3] = nd.w;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sv[e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int off = swz_off<D>(qb * 32 + l32, 2 * kk + hl);
                const bf16x8 aq = *(const bf16x8 *)(Qs + off);
                const bf16x8 ad = *(const bf16x8 *)(dOs + off);
                sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kB[kk], sv, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vB[kk], dp, 0, 0, 0);
            }
            constexpr int A = AHEAD;
            __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
            for (int u = 0; u < 2 * (D / 16) - A; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
            // masked scores become -inf (P = 0) before the exponentials,
            // which then run unconditionally
            if (need_mask) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int qi = q0 + qb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                    const bool vis = (key < Nk) & (qi < Nq) &
                                     (p.noncausal | (key - qi <= p.delta));
                    sv[e] = vis ? sv[e] : -INFINITY;
                }
            }
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int r0 = qb * 32 + gq * 8 + hl * 4;
                const float4 l2 = *(const float4 *)(&lse2s[r0]);
                const float lv[4] = {l2.x, l2.y, l2.z, l2.w};
                float pv[4], dsv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = gq * 4 + u;
                    const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], c, -lv[u]));
                    pv[u] = pe;
                    dsv[u] = pe * dp[e];
                }
                pB[qb][gq * 2 + 0] = pack_bf16(pv[0], pv[1]);
                pB[qb][gq * 2 + 1] = pack_bf16(pv[2], pv[3]);
                dB[qb][gq * 2 + 0] = pack_bf16(dsv[0], dsv[1]);
                dB[qb][gq * 2 + 1] = pack_bf16(dsv[2], dsv[3]);
            }
        }

        // dV^T += dO^T P and dK^T += Q^T dS (k = the tile's BQ query rows)
#pragma unroll
        for (int ks = 0; ks < BQ / 16; ++ks) {
            const int qb = ks >> 1, half = ks & 1;
            u32x4 wp = {pB[qb][half * 4 + 0], pB[qb][half * 4 + 1], pB[qb][half * 4 + 2],
                        pB[qb][half * 4 + 3]};
            u32x4 wd = {dB[qb][half * 4 + 0], dB[qb][half * 4 + 1], dB[qb][half * 4 + 2],
                        dB[qb][half * 4 + 3]};
            const bf16x8 bp = __builtin_bit_cast(bf16x8, wp);
            const bf16x8 bd = __builtin_bit_cast(bf16x8, wd);
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const int cc = 4 * i + 2 * (gg & 1) + ((ip & 3) >> 1);
                const int o0 = swz_off<D>(16 * ks + trow, cc) + (ip & 1) * 8;
                const int o1 = swz_off<D>(16 * ks + 8 + trow, cc) + (ip & 1) * 8;
                const bf16x8 ao = cat_tr(read_tr((const bf16 *)(dOs + o0)), read_tr((const bf16 *)(dOs + o1)));
                const bf16x8 aq = cat_tr(read_tr((const bf16 *)(Qs + o0)), read_tr((const bf16 *)(Qs + o1)));
                accV[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bp, accV[i], 0, 0, 0);
                accK[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bd, accK[i], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
        for (int u = 0; u < 2 * (BQ / 16) * (D / 32) - AHEAD; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
    }

    if (key >= Nk)
        return;
    // accumulated outputs: every running sum is read before any is written,
    // so the reads' round trips overlap instead of following each other
    float4 old[2][D / 32][4];
    if (p.acc_kv) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const View &out = which ? p.dk : p.dv;
            const int64_t krow = b * out.sb + s * out.ss + g * out.sh +
                                 head_shift_elems(out, p.hs_r, hr.off) + (int64_t)key * out.sn;
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    old[which][i][gq] =
                        *(const float4 *)((const float *)out.ptr + krow + i * 32 + gq * 8 + hl * 4);
        }
    }
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const View &out = which ? p.dk : p.dv;
        const int out_f32 = which ? p.dk_f32 : p.dv_f32;
        const float f = which ? p.scale : 1.f;
        const int64_t krow = b * out.sb + s * out.ss + g * out.sh +
                             head_shift_elems(out, p.hs_r, hr.off) + (int64_t)key * out.sn;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = i * 32 + gq * 8 + hl * 4;
                const f32x16 &a = which ? accK[i] : accV[i];
                const float x0 = a[gq * 4 + 0] * f, x1 = a[gq * 4 + 1] * f;
                const float x2 = a[gq * 4 + 2] * f, x3 = a[gq * 4 + 3] * f;
                if (p.acc_kv) {
                    float4 w = old[which][i][gq];
                    w.x += x0; w.y += x1; w.z += x2; w.w += x3;
                    *(float4 *)((float *)out.ptr + krow + d0) = w;
                } else if (out_f32) {
                    float4 w = {x0, x1, x2, x3};
                    *(float4 *)((float *)out.ptr + krow + d0) = w;
                } else {
                    uint2 w = {pack_bf16(x0, x1), pack_bf16(x2, x3)};
                    *(uint2 *)((bf16 *)out.ptr + krow + d0) = w;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dQ, query-tile major: one workgroup = 8 waves = 256 query rows of one
// (batch, query head); wave = 32 rows, whose Q and dO rows are the B operands
// (VGPRs) of S^T = K Q^T and dP^T = V dO^T.  With queries in lane columns, a
// lane holds one row's LSE and D, and dS^T = P^T o (dP^T - D) is directly the
// B operand of dQ^T += K^T dS^T, whose A operand is read from the row-major K
// tile in LDS with transposing reads.  Each (query, d) is owned by one lane,
// so dQ is accumulated without atomics (dq += sigma * dQ at the end).
// ---------------------------------------------------------------------------
constexpr int kQWaves = 8;
constexpr int kQThreads = 64 * kQWaves;
constexpr int kQBQ = 32 * kQWaves;

template <int D>
struct QCfg {
    static constexpr int BK = D == 64 ? 128 : 64;  // keys per tile (same bytes for both d)
    static constexpr int CPT = BK * D / 8 / kQThreads;  // 16-byte chunks per thread per tile
    static_assert(CPT * kQThreads * 8 == BK * D, "tile split");
};

template <int D>
__device__ __forceinline__ void bwd_dq_body(const BwdParams &p, unsigned blk)
{
    using C = QCfg<D>;
    constexpr int BK = C::BK;
    __shared__ __attribute__((aligned(16))) char Ks[BK * 2 * D];
    __shared__ __attribute__((aligned(16))) char Vs[BK * 2 * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int gg = lane >> 4, ip = lane & 15;

    const int nqt = (p.Nq + kQBQ - 1) / kQBQ;
    const int BH = p.B * p.S * p.Hq;
    const WorkItem wi = work_item(blk, nqt, BH, p.grouped_q);
    if (wi.grp >= BH)
        return;  // padding item of a grouped launch
    const int qt = nqt - 1 - wi.t;  // longest first
    const int bsh = wi.grp;
    const int h = bsh % p.Hq, bs = bsh / p.Hq;
    const int s = bs % p.S, b = bs / p.S;
    const int g = (int)(((int64_t)h * p.Hkv) / p.Hq);
    // rows of this head (fewer, and shifted, under head-dependent offsets)
    const HeadRows hr = head_rows(p.hs_r, p.hs_len, p.Nq, h);
    const int Nq = hr.n, Nk = p.hs_r > 0 ? hr.n : p.Nk;
    const int q0 = qt * kQBQ;
    if (q0 >= Nq)
        return;  // past this head's rows

    const bf16 *Q = (const bf16 *)p.q.ptr + b * p.q.sb + s * p.q.ss + h * p.q.sh +
                    head_shift_elems(p.q, p.hs_r, hr.off);
    const bf16 *dO = (const bf16 *)p.dout.ptr + b * p.dout.sb + s * p.dout.ss + h * p.dout.sh +
                     head_shift_elems(p.dout, p.hs_r, hr.off);
    const bf16 *K = (const bf16 *)p.k.ptr + b * p.k.sb + s * p.k.ss + g * p.k.sh +
                    head_shift_elems(p.k, p.hs_r, hr.off);
    const bf16 *V = (const bf16 *)p.v.ptr + b * p.v.sb + s * p.v.ss + g * p.v.sh +
                    head_shift_elems(p.v, p.hs_r, hr.off);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q, ((int64_t)(Nq - 1) * p.q.sn + D) * 2);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(dO, ((int64_t)(Nq - 1) * p.dout.sn + D) * 2);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(K, ((int64_t)(Nk - 1) * p.k.sn + D) * 2);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(V, ((int64_t)(Nk - 1) * p.v.sn + D) * 2);

    const int q0w = q0 + wave * 32;
    const int qrow = q0w + l32;

    int kv_end = Nk;
    if (!p.noncausal)
        kv_end = min(kv_end, max(q0 + kQBQ + p.delta, 0));
    const int ntiles = (kv_end + BK - 1) / BK;
    if (ntiles == 0)
        return;  // no visible key: dq unchanged

    bf16x8 qf[D / 16], of[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        qf[kk] = __builtin_bit_cast(bf16x8, load16(qr, (qrow * (int)p.q.sn + kk * 16 + hl * 8) * 2));
        of[kk] = __builtin_bit_cast(bf16x8, load16(orr, (qrow * (int)p.dout.sn + kk * 16 + hl * 8) * 2));
    }
    float lse2 = INFINITY, dq_d = 0.f;  // +inf: the row contributes P = 0
    if (qrow < Nq) {
        const float lv = *((const float *)p.lse.ptr + b * p.lse.sb + s * p.lse.ss +
                           h * p.lse.sh + head_shift_elems(p.lse, p.hs_r, hr.off) +
                           (int64_t)qrow * p.lse.sn);
        if (lv != -INFINITY)
            lse2 = lv * kLog2e;
        dq_d = *((const float *)p.dvec.ptr + b * p.dvec.sb + s * p.dvec.ss + h * p.dvec.sh +
                 head_shift_elems(p.dvec, p.hs_r, hr.off) + (int64_t)qrow * p.dvec.sn);
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[i][e] = 0.f;
    const float c = p.scale * kLog2e;

    u32x4 kreg[C::CPT], vreg[C::CPT];
    int srow[C::CPT], scol[C::CPT];
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
        const int ch = tid + u * kQThreads;
        srow[u] = ch / (D / 8);
        scol[u] = (ch % (D / 8)) * 8;
    }
    auto load_tile = [&](int t) {
        const int j0 = t * BK;
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            kreg[u] = load16(kr, ((j0 + srow[u]) * (int)p.k.sn + scol[u]) * 2);
            vreg[u] = load16(vr, ((j0 + srow[u]) * (int)p.v.sn + scol[u]) * 2);
        }
    };
    // transposing-read offset of the K^T operand, in the key order of the
    // dS^T accumulator rows
    const int trow = 4 * (gg >> 1) + (ip >> 2);

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            *(u32x4 *)(Ks + swz_off<D>(srow[u], scol[u] >> 3)) = kreg[u];
            *(u32x4 *)(Vs + swz_off<D>(srow[u], scol[u] >> 3)) = vreg[u];
        }
        __syncthreads();
        if (t + 1 < ntiles)
            load_tile(t + 1);

        const int j0 = t * BK;
        if (!p.noncausal && j0 > q0w + 31 + p.delta)
            continue;  // tile entirely in this wave's causal future

        f32x16 s[BK / 32], dp[BK / 32];
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                s[kb][e] = dp[kb][e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int off = swz_off<D>(kb * 32 + l32, 2 * kk + hl);
                const bf16x8 ak = *(const bf16x8 *)(Ks + off);
                const bf16x8 av = *(const bf16x8 *)(Vs + off);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[kk], s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[kk], dp[kb], 0, 0, 0);
            }
        }
        // keep operand reads in flight ahead of the MFMA that uses them
        constexpr int A = D == 64 ? AHEAD : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
        for (int u = 0; u < 2 * (BK / 32) * (D / 16) - A; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
        const bool need_mask = (j0 + BK > Nk) ||
                               (!p.noncausal && j0 + BK - 1 > q0w + p.delta);
        // masked scores become -inf (P = 0) before the exponentials, which
        // then run unconditionally
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = j0 + kb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                    const bool vis = (key < Nk) & (p.noncausal | (key - qrow <= p.delta));
                    s[kb][e] = vis ? s[kb][e] : -INFINITY;
                }
        }
        unsigned pS[BK / 32][8];
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                float ds[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + u], c, -lse2));
                    ds[u] = pe * (dp[kb][e + u] - dq_d);
                }
                pS[kb][e >> 1] = pack_bf16(ds[0], ds[1]);
            }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kb = ks >> 1, half = ks & 1;
            u32x4 w = {pS[kb][half * 4 + 0], pS[kb][half * 4 + 1], pS[kb][half * 4 + 2],
                       pS[kb][half * 4 + 3]};
            const bf16x8 bs = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const int c = 4 * i + 2 * (gg & 1) + ((ip & 3) >> 1);
                const int o0 = swz_off<D>(16 * ks + trow, c) + (ip & 1) * 8;
                const int o1 = swz_off<D>(16 * ks + 8 + trow, c) + (ip & 1) * 8;
                const bf16x8 a = cat_tr(read_tr((const bf16 *)(Ks + o0)), read_tr((const bf16 *)(Ks + o1)));
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs, acc[i], 0, 0, 0);
            }
        }
        // two transposing reads per MFMA; keep four MFMAs' worth in flight
        constexpr int A2 = D == 64 ? AHEAD : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * A2, 0);
#pragma unroll
        for (int u = 0; u < (BK / 16) * (D / 32) - A2; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, A2, 0);
    }

    if (qrow >= Nq)
        return;
    float *dQ = (float *)p.dq.ptr + b * p.dq.sb + s * p.dq.ss + h * p.dq.sh +
                head_shift_elems(p.dq, p.hs_r, hr.off) + (int64_t)qrow * p.dq.sn;
    // every running sum read before any is written (overlapping round trips)
    float4 old[D / 32][4];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
            old[i][gq] = *(const float4 *)(dQ + i * 32 + gq * 8 + hl * 4);
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d0 = i * 32 + gq * 8 + hl * 4;
            float4 x = old[i][gq];
            x.x += p.scale * acc[i][gq * 4 + 0];
            x.y += p.scale * acc[i][gq * 4 + 1];
            x.z += p.scale * acc[i][gq * 4 + 2];
            x.w += p.scale * acc[i][gq * 4 + 3];
            *(float4 *)(dQ + d0) = x;
        }
}

template <int D>
__global__ __launch_bounds__(kQThreads) void bwd_dq_kernel(const BwdParams p)
{
    bwd_dq_body<D>(p, blockIdx.x);
}

// dK/dV and dQ of one segment call in one launch (d = 64): blocks below nkv
// run dK/dV items, blocks from nkv_pad on run dQ items (nkv rounded up to a
// multiple of the XCD count, so both kinds keep their XCD-aware order).  The
// two kinds write different outputs and read only the inputs and D, so they
// may run side by side; one launch fills the chip where either alone would
// not (LongNet's long-segment branches select few rows) and drains once.
template <int D, int BQ, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_kvdq_kernel(const BwdParams p, unsigned nkv,
                                                            unsigned nkv_pad)
{
    static_assert(64 * NW == kQThreads, "both kinds of item use the same workgroup");
    if (blockIdx.x < nkv)
        bwd_kv_body<D, BQ, NW>(p, blockIdx.x);
    else if (blockIdx.x >= nkv_pad)
        bwd_dq_body<D>(p, blockIdx.x - nkv_pad);
}

unsigned zero_grid(int64_t threads)
{
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    return (unsigned)(blocks > 0 ? blocks : 1);
}

}  // namespace

hipError_t launch_bwd_prep(const BwdParams &p, hipStream_t st)
{
    const int64_t rows = (int64_t)p.B * p.S * p.Hq * p.Nq;
    if (rows == 0)
        return hipSuccess;
    int64_t blocks = (rows * 16 + 255) / 256;
    if (blocks > 256 * 64)
        blocks = 256 * 64;  // rows strided over the grid
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_zero_f32(const View &x, int B, int H, int N, int d, hipStream_t st)
{
    const int64_t threads = (int64_t)B * H * N * (d / 4);
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(zero_grid(threads)), dim3(256), 0, st, x, B, H, N, d);
    return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdParams &p0, hipStream_t st)
{
    BwdParams p = p0;
    const int keys = p.d == 128 ? kBKV : 256;
    const int nkt = (p.Nk + keys - 1) / keys;
    const int BSG = p.B * p.S * p.Hkv;
    p.grouped_kv = use_grouped(nkt, BSG);
    const int64_t grid = (int64_t)nkt * BSG == 0 ? 0 : work_items(nkt, BSG, p.grouped_kv);
    if (!grid_fits(grid, kThreads))
        return hipErrorInvalidConfiguration;
    const int nqt = (p.Nq + kQBQ - 1) / kQBQ;
    const int BH = p.B * p.S * p.Hq;
    const bool dq_work = (int64_t)nqt * BH > 0 && p.Nk > 0;
    p.grouped_q = use_grouped(nqt, BH);
    const int64_t qgrid = dq_work ? work_items(nqt, BH, p.grouped_q) : 0;
    if (p.d == 64) {
        const int64_t pad = (grid + kXcds - 1) / kXcds * kXcds;
        if (!grid_fits(pad + qgrid, kQThreads))
            return hipErrorInvalidConfiguration;
        if (pad + qgrid == 0)
            return hipSuccess;
        hipLaunchKernelGGL((bwd_kvdq_kernel<64, kBQ, 8>), dim3((unsigned)(pad + qgrid)),
                           dim3(kQThreads), 0, st, p, (unsigned)grid, (unsigned)pad);
        return hipGetLastError();
    }
    if (grid > 0) {
        hipLaunchKernelGGL(bwd_main_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, st, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (!dq_work)
        return hipSuccess;
    if (!grid_fits(qgrid, kQThreads))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)qgrid), dim3(kQThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace seqattn
