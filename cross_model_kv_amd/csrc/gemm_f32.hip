// The map for fp32 caches (all-fp32 configurations): the same computation as the bf16
// matrix-core path, on the vector ALUs in fp32, for small caches where the exact fp32
// result matters more than throughput.  One workgroup maps 64 tokens of one target head:
//   Y[p, e] = sum_f X[p, f] * W[t][h*d + e][f] + b[t][h*d + e],  then target RoPE (keys).
// A thread owns 4 tokens x d/16 output columns spaced 16 apart, so both members
// (e, e + d/2) of every RoPE pair are in the same thread.

#include "common.h"
#include "internal.h"

namespace kvmap {

template <int D>
__global__ __launch_bounds__(256) void map_f32_kernel(MapArgs a, int L_tgt, int H, int k,
                                                      int64_t T, int nPB) {
    constexpr int TP = 64;       // tokens per workgroup
    constexpr int KS = 16;       // features per step
    constexpr int CN = D / 16;   // output columns per thread
    constexpr int HALF = D / 2;
    __shared__ float Xs[KS][TP + 1];
    __shared__ float Ws[KS][D + 1];

    int b = blockIdx.x;
    const int pb = b % nPB; b /= nPB;
    const int h = b % H; b /= H;
    const int kv = b & 1;
    const int t = b >> 1;
    if (t >= L_tgt) return;

    const int N = H * D, F = k * N;
    const int tid = threadIdx.x;
    const int tp = tid >> 4, tn = tid & 15;
    const int64_t p0 = (int64_t)pb * TP;
    const float* __restrict__ X = (const float*)(kv ? a.xv : a.xk);
    const float* __restrict__ W = (const float*)(kv ? a.Wv : a.Wk) + ((size_t)t * N + (size_t)h * D) * F;
    const int32_t* __restrict__ sel = a.sel + t * k;

    float acc[4][CN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < CN; ++c) acc[r][c] = 0.f;

    for (int k0 = 0; k0 < F; k0 += KS) {
        const int s = k0 / D, e0 = k0 - s * D;
        const int j = s / H, hs = s - j * H;
        const float* xs = X + (((size_t)sel[j] * H + hs) * T) * D + e0;
#pragma unroll
        for (int u = 0; u < (TP * KS) / 256; ++u) {
            const int idx = tid + 256 * u;
            const int row = idx / KS, f = idx % KS;
            const int64_t p = min(p0 + row, T - 1);
            Xs[f][row] = xs[p * D + f];
        }
#pragma unroll
        for (int u = 0; u < (D * KS) / 256; ++u) {
            const int idx = tid + 256 * u;
            const int o = idx / KS, f = idx % KS;
            Ws[f][o] = W[(size_t)o * F + k0 + f];
        }
        __syncthreads();
#pragma unroll
        for (int f = 0; f < KS; ++f) {
            float xr[4], wr[CN];
#pragma unroll
            for (int r = 0; r < 4; ++r) xr[r] = Xs[f][tp * 4 + r];
#pragma unroll
            for (int c = 0; c < CN; ++c) wr[c] = Ws[f][tn + 16 * c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < CN; ++c) acc[r][c] = fmaf(xr[r], wr[c], acc[r][c]);
        }
        __syncthreads();
    }

    const float* __restrict__ bias = (const float*)(kv ? a.bv : a.bk) + (size_t)t * N + (size_t)h * D;
    float* __restrict__ out = (float*)(kv ? a.outv : a.outk);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t p = p0 + tp * 4 + r;
        if (p >= T) continue;
        float y[CN];
#pragma unroll
        for (int c = 0; c < CN; ++c) y[c] = acc[r][c] + bias[tn + 16 * c];
        if (kv == 0) {
#pragma unroll
            for (int c = 0; c < CN / 2; ++c) {
                const int e = tn + 16 * c;
                const float2 cs = a.tab_tgt[p * HALF + e];
                const float lo = y[c], hi = y[c + CN / 2];
                y[c] = fmaf(-hi, cs.y, lo * cs.x);
                y[c + CN / 2] = fmaf(lo, cs.y, hi * cs.x);
            }
        }
        float* o = out + (((size_t)t * H + h) * T + p) * D;
#pragma unroll
        for (int c = 0; c < CN; ++c) o[tn + 16 * c] = y[c];
    }
}

hipError_t launch_map_f32(const MapArgs& a, const ApplyGeom& g, hipStream_t s) {
    const int nPB = (int)((g.T + 63) / 64);
    const int64_t blocks = (int64_t)nPB * g.H * 2 * g.L_tgt;
    if (g.d == 128)
        hipLaunchKernelGGL(map_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a, g.L_tgt, g.H, g.k, g.T, nPB);
    else
        hipLaunchKernelGGL(map_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, g.L_tgt, g.H, g.k, g.T, nPB);
    return hipGetLastError();
}

}  // namespace kvmap
