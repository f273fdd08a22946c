// Log-sum-exp merge of partial attention results, and small helpers.
//
// Exact segment-by-segment attention ("Ultra-Long Sequence Distributed
// Transformer", Abstract: a partial self-attention per segment) is recovered
// by weighting each partial with its share of the softmax normaliser:
//   M = max(La, Lb), wa = e^(La-M), wb = e^(Lb-M),
//   O = (wa Oa + wb Ob) / (wa + wb),  L = M + ln(wa + wb),
// with (0, -inf) as the empty partial.  The merge is bound by HBM bandwidth:
// each thread moves 16-byte vectors of one row, a row's threads sit in one
// wavefront so the row's LSE is read once per lane and written by the first.
#include "common.h"

namespace seqattn {
namespace {

typedef __bf16 bf16;

__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams p)
{
    const int tpr = p.d / 4;  // threads per row (float4 each)
    const int64_t total = (int64_t)p.B * p.H * p.N * tpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += stride) {
        const int64_t row = gid / tpr;
        const int c4 = (int)(gid % tpr) * 4;
        const int n = (int)(row % p.N);
        const int64_t bh = row / p.N;
        const int h = (int)(bh % p.H), b = (int)(bh / p.H);
        float *La = (float *)p.la.ptr + b * p.la.sb + h * p.la.sh + (int64_t)n * p.la.sn;
        const float lb = *((const float *)p.lb.ptr + b * p.lb.sb + h * p.lb.sh + (int64_t)n * p.lb.sn);
        float *Oa = (float *)p.oa.ptr + b * p.oa.sb + h * p.oa.sh + (int64_t)n * p.oa.sn + c4;
        const int64_t ob_off = b * p.ob.sb + h * p.ob.sh + (int64_t)n * p.ob.sn + c4;
        const float la = *La;
        const float M = fmaxf(la, lb);
        if (M == -INFINITY) {
            float4 z = {0.f, 0.f, 0.f, 0.f};
            *(float4 *)Oa = z;
            continue;  // LSE stays -inf
        }
        const float wa = __expf(la - M), wb = __expf(lb - M);
        const float tot = wa + wb;
        const float fa = wa / tot, fb = wb / tot;
        float4 xb;
        if (p.ob_f32) {
            xb = *(const float4 *)((const float *)p.ob.ptr + ob_off);
        } else {
            const uint2 raw = *(const uint2 *)((const bf16 *)p.ob.ptr + ob_off);
            xb.x = __uint_as_float(raw.x << 16);
            xb.y = __uint_as_float(raw.x & 0xffff0000u);
            xb.z = __uint_as_float(raw.y << 16);
            xb.w = __uint_as_float(raw.y & 0xffff0000u);
        }
        float4 xa = *(float4 *)Oa;
        xa.x = fa * xa.x + fb * xb.x;
        xa.y = fa * xa.y + fb * xb.y;
        xa.z = fa * xa.z + fb * xb.z;
        xa.w = fa * xa.w + fb * xb.w;
        *(float4 *)Oa = xa;
        if (c4 == 0)
            *La = M + __logf(tot);
    }
}

// (O, LSE) <- (0, -inf) over a [B][S][H][N] view
__global__ __launch_bounds__(256) void fill_empty_kernel(View o, View lse, int B, int S,
                                                         int H, int N, int d, int o_f32)
{
    const int tpr = d / 4;
    const int64_t total = (int64_t)B * S * H * N * tpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += stride) {
        const int64_t row = gid / tpr;
        const int c4 = (int)(gid % tpr) * 4;
        const int n = (int)(row % N);
        int64_t r = row / N;
        const int h = (int)(r % H);
        r /= H;
        const int s = (int)(r % S), b = (int)(r / S);
        const int64_t off = b * o.sb + s * o.ss + h * o.sh + (int64_t)n * o.sn + c4;
        if (o_f32) {
            float4 z = {0.f, 0.f, 0.f, 0.f};
            *(float4 *)((float *)o.ptr + off) = z;
        } else {
            uint2 z = {0u, 0u};
            *(uint2 *)((bf16 *)o.ptr + off) = z;
        }
        if (c4 == 0)
            *((float *)lse.ptr + b * lse.sb + s * lse.ss + h * lse.sh + (int64_t)n * lse.sn) =
                -INFINITY;
    }
}

__device__ inline unsigned pack2(float a, float b)
{
    bf16 x = (bf16)a, y = (bf16)b;
    return (unsigned)__builtin_bit_cast(unsigned short, x) |
           ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(View src, View dst, int B, int H,
                                                        int N, int d)
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
        const float4 x = *(const float4 *)((const float *)src.ptr + b * src.sb + h * src.sh +
                                           (int64_t)n * src.sn + c4);
        uint2 w = {pack2(x.x, x.y), pack2(x.z, x.w)};
        *(uint2 *)((bf16 *)dst.ptr + b * dst.sb + h * dst.sh + (int64_t)n * dst.sn + c4) = w;
    }
}

unsigned grid_for(int64_t threads)
{
    int64_t blocks = (threads + 255) / 256;
    const int64_t cap = 256 * 64;  // enough resident waves to saturate HBM
    if (blocks > cap)
        blocks = cap;
    return (unsigned)(blocks > 0 ? blocks : 1);
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t st)
{
    const int64_t threads = (int64_t)p.B * p.H * p.N * (p.d / 4);
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(grid_for(threads)), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_fill_empty(const View &o, const View &lse, int B, int S, int H, int N,
                             int d, int o_f32, hipStream_t st)
{
    const int64_t threads = (int64_t)B * S * H * N * (d / 4);
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(fill_empty_kernel, dim3(grid_for(threads)), dim3(256), 0, st, o, lse,
                       B, S, H, N, d, o_f32);
    return hipGetLastError();
}

hipError_t launch_cast_bf16(const View &src, const View &dst, int B, int H, int N, int d,
                            hipStream_t st)
{
    const int64_t threads = (int64_t)B * H * N * (d / 4);
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(threads)), dim3(256), 0, st, src, dst,
                       B, H, N, d);
    return hipGetLastError();
}

}  // namespace seqattn
