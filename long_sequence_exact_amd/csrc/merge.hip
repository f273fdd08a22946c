// Log-sum-exp merge of partial attention results, and small helpers.
//
// Exact segment-by-segment attention ("Ultra-Long Sequence Distributed
// Transformer", Abstract: a partial self-attention per segment) is recovered
// by weighting each partial with its share of the softmax normaliser:
//   M = max(La, Lb), wa = e^(La-M), wb = e^(Lb-M),
//   O = (wa Oa + wb Ob) / (wa + wb),  L = M + ln(wa + wb),
// with (0, -inf) as the empty partial.  The merge is bound by HBM bandwidth:
// each thread moves 16-byte vectors of one row, a row's threads sit in one
// wavefront so the row's LSE is read by each of its lanes (one request) and
// written by the first.
#include "common.h"

namespace seqattn {
namespace {

typedef __bf16 bf16;

// Each thread merges 8 consecutive elements of one row (two 16-byte vectors
// of the fp32 accumulator, 32 or 16 bytes of the partial), so a wave keeps
// enough bytes in flight to cover HBM latency; a row's d/8 threads are
// consecutive lanes of one wave.
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams p)
{
    const int tpr = p.d / 8;  // threads per row
    const int64_t total = (int64_t)p.B * p.H * p.N * tpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += stride) {
        const int64_t row = gid / tpr;
        const int c8 = (int)(gid % tpr) * 8;
        const int n = (int)(row % p.N);
        const int64_t bh = row / p.N;
        const int h = (int)(bh % p.H), b = (int)(bh / p.H);
        float *La = (float *)p.la.ptr + b * p.la.sb + h * p.la.sh + (int64_t)n * p.la.sn;
        const float lb = *((const float *)p.lb.ptr + b * p.lb.sb + h * p.lb.sh + (int64_t)n * p.lb.sn);
        float *Oa = (float *)p.oa.ptr + b * p.oa.sb + h * p.oa.sh + (int64_t)n * p.oa.sn + c8;
        const int64_t ob_off = b * p.ob.sb + h * p.ob.sh + (int64_t)n * p.ob.sn + c8;
        const float la = *La;
        float4 xa0 = *(const float4 *)Oa, xa1 = *(const float4 *)(Oa + 4);
        float4 xb0, xb1;
        if (p.ob_f32) {
            xb0 = *(const float4 *)((const float *)p.ob.ptr + ob_off);
            xb1 = *(const float4 *)((const float *)p.ob.ptr + ob_off + 4);
        } else {
            const uint4 raw = *(const uint4 *)((const bf16 *)p.ob.ptr + ob_off);
            xb0.x = __uint_as_float(raw.x << 16);
            xb0.y = __uint_as_float(raw.x & 0xffff0000u);
            xb0.z = __uint_as_float(raw.y << 16);
            xb0.w = __uint_as_float(raw.y & 0xffff0000u);
            xb1.x = __uint_as_float(raw.z << 16);
            xb1.y = __uint_as_float(raw.z & 0xffff0000u);
            xb1.z = __uint_as_float(raw.w << 16);
            xb1.w = __uint_as_float(raw.w & 0xffff0000u);
        }
        const float M = fmaxf(la, lb);
        float fa = 0.f, fb = 0.f, lnew = -INFINITY;
        if (M != -INFINITY) {  // else both partials are empty: (0, -inf)
            const float wa = __expf(la - M), wb = __expf(lb - M);
            const float tot = wa + wb;
            fa = wa / tot;
            fb = wb / tot;
            lnew = M + __logf(tot);
        }
        if (M == -INFINITY) {  // O of an empty result is 0 whatever the inputs held
            xa0 = xa1 = xb0 = xb1 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        xa0.x = fa * xa0.x + fb * xb0.x;
        xa0.y = fa * xa0.y + fb * xb0.y;
        xa0.z = fa * xa0.z + fb * xb0.z;
        xa0.w = fa * xa0.w + fb * xb0.w;
        xa1.x = fa * xa1.x + fb * xb1.x;
        xa1.y = fa * xa1.y + fb * xb1.y;
        xa1.z = fa * xa1.z + fb * xb1.z;
        xa1.w = fa * xa1.w + fb * xb1.w;
        *(float4 *)Oa = xa0;
        *(float4 *)(Oa + 4) = xa1;
        if (c8 == 0)
            *La = lnew;
    }
}

__device__ inline unsigned pack2(float a, float b)
{
    bf16 x = (bf16)a, y = (bf16)b;
    return (unsigned)__builtin_bit_cast(unsigned short, x) |
           ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

// The key-range chunks of a split segment forward merged into its output:
// for row n, the chunks its query tile computed (the parts of the tile's
// visible key range, as the forward cuts it) are combined by their
// log-sum-exp; a row with none gets (0, -inf).  One thread per 8 elements of
// a row, as in lse_merge_kernel.
__global__ __launch_bounds__(256) void chunk_merge_kernel(const ChunkMergeParams p)
{
    const int tpr = p.d / 8;
    const int64_t total = (int64_t)p.B * p.H * p.N * tpr;
    const int64_t bhn = (int64_t)p.B * p.H * p.N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += stride) {
        const int64_t row = gid / tpr;  // [B][H][N] row of the partials
        const int c8 = (int)(gid % tpr) * 8;
        const int n = (int)(row % p.N);
        const int64_t bh = row / p.N;
        const int h = (int)(bh % p.H), b = (int)(bh / p.H);
        int kv_end = p.Nk;
        if (!p.noncausal) {
            const int tile = n / p.tile_rows;
            kv_end = min(kv_end, max((tile + 1) * p.tile_rows + p.delta, 0));
        }
        // the forward's parts of this tile's visible keys (same rule)
        const int len = max(p.kv_chunk, ((kv_end + p.nchunk - 1) / p.nchunk + 255) / 256 * 256);
        const int nc = min(p.nchunk, (kv_end + len - 1) / len);
        float lc[8];  // static indices only (registers)
        float M = -INFINITY;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            lc[c] = -INFINITY;
            if (c < nc)
                lc[c] = p.pl[c * bhn + row];
            M = fmaxf(M, lc[c]);
        }
        float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
        float tot = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (c >= nc)
                    break;
                const float w = __expf(lc[c] - M);
                const float *src = p.po + (c * bhn + row) * p.d + c8;
                const float4 x0 = *(const float4 *)src, x1 = *(const float4 *)(src + 4);
                tot += w;
                a0.x += w * x0.x; a0.y += w * x0.y; a0.z += w * x0.z; a0.w += w * x0.w;
                a1.x += w * x1.x; a1.y += w * x1.y; a1.z += w * x1.z; a1.w += w * x1.w;
            }
            const float inv = 1.f / tot;
            a0.x *= inv; a0.y *= inv; a0.z *= inv; a0.w *= inv;
            a1.x *= inv; a1.y *= inv; a1.z *= inv; a1.w *= inv;
        }
        const int64_t off = b * p.o.sb + h * p.o.sh + (int64_t)n * p.o.sn + c8;
        if (p.o_f32) {
            *(float4 *)((float *)p.o.ptr + off) = a0;
            *(float4 *)((float *)p.o.ptr + off + 4) = a1;
        } else {
            uint4 w;
            w.x = pack2(a0.x, a0.y);
            w.y = pack2(a0.z, a0.w);
            w.z = pack2(a1.x, a1.y);
            w.w = pack2(a1.z, a1.w);
            *(uint4 *)((bf16 *)p.o.ptr + off) = w;
        }
        if (c8 == 0)
            *((float *)p.lse.ptr + b * p.lse.sb + h * p.lse.sh + (int64_t)n * p.lse.sn) =
                M == -INFINITY ? -INFINITY : M + __logf(tot);
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
    // one work item per thread up to 2^26 threads: a grid-stride loop over
    // several items per thread measured 5-7% slower on the merge
    const int64_t cap = 256 * 1024;
    if (blocks > cap)
        blocks = cap;
    return (unsigned)(blocks > 0 ? blocks : 1);
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t st)
{
    const int64_t threads = (int64_t)p.B * p.H * p.N * (p.d / 8);
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(grid_for(threads)), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_chunk_merge(const ChunkMergeParams &p, hipStream_t st)
{
    const int64_t threads = (int64_t)p.B * p.H * p.N * (p.d / 8);
    if (threads == 0)
        return hipSuccess;
    if (p.nchunk < 1 || p.nchunk > 8 || p.d % 8 != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(chunk_merge_kernel, dim3(grid_for(threads)), dim3(256), 0, st, p);
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
