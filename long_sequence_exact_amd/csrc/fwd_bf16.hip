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
//     SIMD, so one wave's softmax VALU work overlaps the other's MFMAs;
//   * the workgroup walks the KV segment in tiles of BK keys (64 for d=128,
//     128 for d=64), staged HBM -> VGPR -> LDS; the next tile's global loads
//     are issued before the current tile is computed;
//   * per tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//     (K from LDS as the A operand, Q held in VGPRs as the B operand), so the
//     accumulator puts one query row in one lane column: the row max needs a
//     single cross-lane step (lane l <-> l^32) and the row sum none until the
//     epilogue;
//   * the reference max of a row is only raised when new scores exceed it by
//     more than 2^8 (a conditional rescale): the exponentials stay <= 256,
//     which fp32 and bf16 hold with full relative precision, and the O
//     rescale is skipped for most tiles;
//   * P^T is rounded to bf16 in registers and is directly the B operand of
//     O^T += V^T P^T; V is transposed while it is written to LDS, in a key
//     order that matches the accumulator's row interleave;
//   * causal tiles above the diagonal are never visited; only tiles that
//     straddle it (or the segment tail) are masked;
//   * workgroups are issued longest-first (last query tile first) with the
//     (batch, segment, head) index fastest, so consecutive workgroups -- which
//     the dispatcher spreads round-robin over the 8 XCDs -- stream the same
//     K/V tiles at about the same time.
#include "common.h"

namespace seqattn {
namespace {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kWaves = 8;
constexpr int kBQ = 32 * kWaves;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 headroom before the max is raised

template <int D>
struct Cfg {
    static constexpr int BK = (D == 128) ? 64 : 128;  // keys per tile
    static constexpr int KSTR = D + 8;                // K row pitch in LDS (bf16)
    static constexpr int VSTR = BK + 8;               // V^T row pitch in LDS (bf16)
    static constexpr int KCH = BK * D / 8 / kThreads; // 16-byte K chunks per thread
    static constexpr int VG = BK / 4;                 // 4-key groups per tile
    static constexpr int VBLK = VG * (D / 8);        // 4x8 V blocks per tile
    static_assert(VBLK <= kThreads && BK * D / 8 == KCH * kThreads, "staging split");
};

__device__ inline unsigned pack_bf16(float a, float b)
{
    // round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950)
    bf16 x = (bf16)a, y = (bf16)b;
    return (unsigned)__builtin_bit_cast(unsigned short, x) |
           ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

// Position of key group (4 keys starting at 4*kg) inside the permuted V^T row:
// within every 16 keys the order is [0-3, 8-11, 4-7, 12-15], so that lane half
// 0 of the PV MFMA reads keys {0-3, 8-11} and half 1 keys {4-7, 12-15} as one
// 16-byte chunk -- the same keys the S^T accumulator gives each lane half.
__device__ inline int vt_pos(int kg)
{
    const int q4 = kg & 3;
    return (kg >> 2) * 16 + (((q4 & 1) << 1) | (q4 >> 1)) * 4;
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(const FwdParams p)
{
    using C = Cfg<D>;
    constexpr int BK = C::BK;
    __shared__ __attribute__((aligned(16))) bf16 Ks[BK * C::KSTR];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D * C::VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    const int nqt = (p.Nq + kBQ - 1) / kBQ;
    const int BH = p.B * p.S * p.Hq;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const int h = bh % p.Hq;
    const int bs = bh / p.Hq;
    const int s = bs % p.S, b = bs / p.S;
    const int g = (int)(((int64_t)h * p.Hkv) / p.Hq);

    const bf16 *Q = (const bf16 *)p.q.ptr + b * p.q.sb + s * p.q.ss + h * p.q.sh;
    const bf16 *K = (const bf16 *)p.k.ptr + b * p.k.sb + s * p.k.ss + g * p.k.sh;
    const bf16 *V = (const bf16 *)p.v.ptr + b * p.v.sb + s * p.v.ss + g * p.v.sh;

    const int q0 = qt * kBQ;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + l32;

    int kv_end = p.Nk;
    if (!p.noncausal) {
        const int lim = q0 + kBQ + p.delta;  // keys < lim can be visible
        kv_end = min(kv_end, max(lim, 0));
    }
    const int ntiles = (kv_end + BK - 1) / BK;

    if (ntiles == 0 && p.accumulate)
        return;  // empty partial: the running accumulator is unchanged

    // Q tile as the B operand of S^T = K Q^T: lane (l32, hl) holds row qrow,
    // d = 16*kk + 8*hl .. +8.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qrow < p.Nq)
            raw = *(const u32x4 *)(Q + (int64_t)qrow * p.q.sn + kk * 16 + hl * 8);
        qf[kk] = __builtin_bit_cast(bf16x8, raw);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oacc[i][e] = 0.f;

    float m_run = -INFINITY;  // running max, in units of log2
    float l_run = 0.f;        // this lane's partial row sum
    const float c = p.scale * kLog2e;

    u32x4 kreg[C::KCH];
    u32x4 vreg[4];
    const bool vthread = tid < C::VBLK;  // threads 0..VBLK-1 also stage one V block
    const int vkg = tid % C::VG, vdc = (tid / C::VG) % (D / 8);

    auto load_tile = [&](int t) {
        const int j0 = t * BK;
#pragma unroll
        for (int u = 0; u < C::KCH; ++u) {
            const int ch = tid + u * kThreads;
            const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
            const int j = j0 + row;
            u32x4 z = {0u, 0u, 0u, 0u};
            kreg[u] = (j < p.Nk) ? *(const u32x4 *)(K + (int64_t)j * p.k.sn + col) : z;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + vkg * 4 + u;
            u32x4 z = {0u, 0u, 0u, 0u};
            vreg[u] = (vthread && j < p.Nk) ? *(const u32x4 *)(V + (int64_t)j * p.v.sn + vdc * 8) : z;
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < C::KCH; ++u) {
            const int ch = tid + u * kThreads;
            const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
            *(u32x4 *)(&Ks[row * C::KSTR + col]) = kreg[u];
        }
        // 4 keys x 8 d block -> 8 rows of V^T, 4 keys (8 bytes) each
        if (!vthread)
            return;
        const int pos = vt_pos(vkg);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const unsigned a0 = vreg[0][m], a1 = vreg[1][m], a2 = vreg[2][m], a3 = vreg[3][m];
            uint2 lo, hi;
            lo.x = (a0 & 0xffffu) | (a1 << 16);
            lo.y = (a2 & 0xffffu) | (a3 << 16);
            hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
            hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
            *(uint2 *)(&Vt[(vdc * 8 + 2 * m) * C::VSTR + pos]) = lo;
            *(uint2 *)(&Vt[(vdc * 8 + 2 * m + 1) * C::VSTR + pos]) = hi;
        }
    };

    if (ntiles > 0)
        load_tile(0);

    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();  // every wave is done reading the previous tile
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles)
            load_tile(t + 1);

        const int j0 = t * BK;
        // whole tile invisible to this wave's rows (causal diagonal): skip
        if (!p.noncausal && j0 > q0w + 31 + p.delta)
            continue;

        f32x16 sacc[BK / 32];
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const bf16x8 a = *(const bf16x8 *)(&Ks[(kb * 32 + l32) * C::KSTR + kk * 16 + hl * 8]);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kb], 0, 0, 0);
            }
        }

        // accumulator element e of block kb: key j0 + 32kb + 8(e/4) + 4hl + e%4,
        // query qrow
        const bool need_mask = (j0 + BK > p.Nk) ||
                               (!p.noncausal && j0 + BK - 1 > q0w + p.delta);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = j0 + kb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                    const bool vis = key < p.Nk && (p.noncausal || key - qrow <= p.delta);
                    if (!vis)
                        sacc[kb][e] = -INFINITY;
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                mx = fmaxf(mx, sacc[kb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));

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

        unsigned pk[BK / 32][8];
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], c, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e + 1], c, -m_use));
                lsum += p0 + p1;
                pk[kb][e >> 1] = pack_bf16(p0, p1);
            }
        l_run = l_run * alpha + lsum;

#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kb = ks >> 1, half = ks & 1;
            u32x4 pw = {pk[kb][half * 4 + 0], pk[kb][half * 4 + 1],
                        pk[kb][half * 4 + 2], pk[kb][half * 4 + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const bf16x8 a = *(const bf16x8 *)(&Vt[(i * 32 + l32) * C::VSTR + ks * 16 + hl * 8]);
                oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[i], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l), optional merge ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool has = l_tot > 0.f;
    const float inv = has ? 1.f / l_tot : 0.f;
    const float lse_new = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (qrow >= p.Nq)
        return;

    float *Lp = (float *)p.lse.ptr + b * p.lse.sb + s * p.lse.ss + h * p.lse.sh +
                (int64_t)qrow * p.lse.sn;
    const int64_t orow = b * p.o.sb + s * p.o.ss + h * p.o.sh + (int64_t)qrow * p.o.sn;

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

    // fused merge with the running fp32 partial (o, lse)
    const float la = *Lp;
    const float M = fmaxf(la, lse_new);
    if (M == -INFINITY)
        return;  // both empty: stays (0, -inf)
    const float wa = __expf(la - M), wb = __expf(lse_new - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb / tot * inv;
    float *Op = (float *)p.o.ptr + orow;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d0 = i * 32 + gq * 8 + hl * 4;
            float4 a = *(float4 *)(Op + d0);
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

hipError_t launch_fwd_bf16(const FwdParams &p, int d, hipStream_t st)
{
    const int nqt = (p.Nq + kBQ - 1) / kBQ;
    const int64_t grid = (int64_t)nqt * p.B * p.S * p.Hq;
    if (grid == 0)
        return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, st, p);
    else
        hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace seqattn
