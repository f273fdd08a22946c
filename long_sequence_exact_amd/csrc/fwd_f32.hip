// Segment forward, fp32 inputs (VALU path).
//
// Same contract as the bf16 MFMA kernel -- partial attention of a query block
// against one KV segment with optional fused log-sum-exp merge ("Ultra-Long
// Sequence Distributed Transformer", Abstract) -- for callers that keep
// Q/K/V in fp32.  gfx950 has no fp32 matrix path worth the layout work at
// the sizes fp32 is used for, so one thread owns one query row: q and the
// output row live in VGPRs, K/V tiles of 32 keys are staged through LDS and
// read as broadcasts, and the softmax is the exact online recurrence in fp32.
#include "common.h"

namespace seqattn {
namespace {

constexpr int kRows = 64;  // query rows (threads) per workgroup
constexpr int kTK = 32;    // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(const FwdParams p)
{
    __shared__ float Ks[kTK][D];
    __shared__ float Vs[kTK][D];

    const int tid = threadIdx.x;
    const int nqt = (p.Nq + kRows - 1) / kRows;
    const int BH = p.B * p.S * p.Hq;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const int h = bh % p.Hq;
    const int bs = bh / p.Hq;
    const int s = bs % p.S, b = bs / p.S;
    const int g = (int)(((int64_t)h * p.Hkv) / p.Hq);

    const float *Q = (const float *)p.q.ptr + b * p.q.sb + s * p.q.ss + h * p.q.sh;
    const float *K = (const float *)p.k.ptr + b * p.k.sb + s * p.k.ss + g * p.k.sh;
    const float *V = (const float *)p.v.ptr + b * p.v.sb + s * p.v.ss + g * p.v.sh;

    const int q0 = qt * kRows;
    const int qrow = q0 + tid;
    int kv_end = p.Nk;
    if (!p.noncausal)
        kv_end = min(kv_end, max(q0 + kRows + p.delta, 0));
    if (kv_end == 0 && p.accumulate)
        return;

    float q[D], o[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = (qrow < p.Nq) ? Q[(int64_t)qrow * p.q.sn + c] : 0.f;
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    for (int j0 = 0; j0 < kv_end; j0 += kTK) {
        __syncthreads();
        for (int x = tid; x < kTK * D; x += kRows) {
            const int r = x / D, c = x % D;
            const int j = j0 + r;
            Ks[r][c] = (j < p.Nk) ? K[(int64_t)j * p.k.sn + c] : 0.f;
            Vs[r][c] = (j < p.Nk) ? V[(int64_t)j * p.v.sn + c] : 0.f;
        }
        __syncthreads();
        for (int r = 0; r < kTK; ++r) {
            const int j = j0 + r;
            if (j >= p.Nk || (!p.noncausal && j - qrow > p.delta))
                continue;
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c)
                dot = __builtin_fmaf(q[c], Ks[r][c], dot);
            const float sc = dot * p.scale;
            if (sc > m) {
                const float corr = expf(m - sc);
                l *= corr;
#pragma unroll
                for (int c = 0; c < D; ++c)
                    o[c] *= corr;
                m = sc;
            }
            const float pj = expf(sc - m);
            l += pj;
#pragma unroll
            for (int c = 0; c < D; ++c)
                o[c] = __builtin_fmaf(pj, Vs[r][c], o[c]);
        }
    }

    if (qrow >= p.Nq)
        return;
    const bool has = l > 0.f;
    const float inv = has ? 1.f / l : 0.f;
    const float lse_new = has ? m + logf(l) : -INFINITY;
    float *Lp = (float *)p.lse.ptr + b * p.lse.sb + s * p.lse.ss + h * p.lse.sh +
                (int64_t)qrow * p.lse.sn;
    float *Op = (float *)p.o.ptr + b * p.o.sb + s * p.o.ss + h * p.o.sh +
                (int64_t)qrow * p.o.sn;
    if (!p.accumulate) {
#pragma unroll
        for (int c = 0; c < D; ++c)
            Op[c] = o[c] * inv;
        *Lp = lse_new;
        return;
    }
    const float la = *Lp;
    const float M = fmaxf(la, lse_new);
    if (M == -INFINITY)
        return;
    const float wa = expf(la - M), wb = expf(lse_new - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb / tot * inv;
#pragma unroll
    for (int c = 0; c < D; ++c)
        Op[c] = fa * Op[c] + fb * o[c];
    *Lp = M + logf(tot);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams &p, int d, hipStream_t st)
{
    const int nqt = (p.Nq + kRows - 1) / kRows;
    const int64_t grid = (int64_t)nqt * p.B * p.S * p.Hq;
    if (grid == 0)
        return hipSuccess;
    if (!grid_fits(grid, kRows))
        return hipErrorInvalidConfiguration;
    if (d == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(kRows), 0, st, p);
    else
        hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(kRows), 0, st, p);
    return hipGetLastError();
}

}  // namespace seqattn
