// RoPE tables and the key de-rotation producer.
//
// Half-split rotary encoding: pair (i, i + d/2) of a key at absolute position p is
// rotated by a = p * theta^(-2i/d).  The mapper works in content space: source keys are
// rotated back by -a with the source model's factors before the map, and mapped keys are
// rotated forward with the target model's factors afterwards (VeloxQuant-MLX "Cross-Model
// KV Transfer", section "The mapping", item 3; KVBridge README, "What ships": exact
// inverse/forward RoPE using each model's factors).
//
// Angles are formed and evaluated in float64 and only the cos/sin are stored in fp32:
// an fp32 product p * f_i is off by ~1e-3 rad at p = 32767, the size of deviation the
// VeloxQuant-MLX "Metal kernel" section reports for its fp32 path.

#include "common.h"
#include "internal.h"

namespace kvmap {

__device__ __forceinline__ double rope_freq(const RopeFreqs& fr, int i, int d) {
    return fr.given ? fr.f[i] : pow(fr.theta, -2.0 * (double)i / (double)d);
}

__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int64_t T, int d,
                                                         const RopeFreqs fr, int64_t pos0) {
    const int half = d / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * half) return;
    const int64_t t = idx / half;
    const int i = (int)(idx - t * half);
    const double a = (double)(pos0 + t) * rope_freq(fr, i, d);
    double s, c;
    sincos(a, &s, &c);
    tab[idx] = make_float2((float)c, (float)s);
}

// Recode table: (cos A, sin A) with A = (pos0_s + t) f_s,i - (pos0_t + t) f_t,i, formed in
// float64 (the two products reach ~3e4 rad at 32K positions; their difference in fp32 would
// be off by ~1e-3).  Rotating a source-roped key by -A strips the source RoPE and applies the
// target one in a single rotation (VeloxQuant-MLX "Cross-Model KV Transfer", section "Metal
// kernel": the strip and the target rotation turn one pair at one position, so they compose).
__global__ __launch_bounds__(256) void rope_diff_table_kernel(float2* __restrict__ tab, int64_t T, int d,
                                                              const RopeFreqs fs, int64_t pos0_s,
                                                              const RopeFreqs ft, int64_t pos0_t) {
    const int half = d / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * half) return;
    const int64_t t = idx / half;
    const int i = (int)(idx - t * half);
    const double a = (double)(pos0_s + t) * rope_freq(fs, i, d) - (double)(pos0_t + t) * rope_freq(ft, i, d);
    double s, c;
    sincos(a, &s, &c);
    tab[idx] = make_float2((float)c, (float)s);
}

hipError_t launch_rope_diff_table(float2* tab, int64_t T, int d, const RopeFreqs& fs, int64_t pos0_s,
                                  const RopeFreqs& ft, int64_t pos0_t, hipStream_t s) {
    const int64_t n = T * (d / 2);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(rope_diff_table_kernel, dim3(blocks), dim3(256), 0, s, tab, T, d, fs, pos0_s, ft, pos0_t);
    return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int64_t T, int d, const RopeFreqs& fr, int64_t pos0, hipStream_t s) {
    const int64_t n = T * (d / 2);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, tab, T, d, fr, pos0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Producer: one pass over every selected source key layer, reading each element once with
// 16-byte coalesced loads.  A thread owns VEC consecutive pairs (i .. i+VEC-1) of one token
// row: it loads the matching VEC elements of the low half and of the high half, keeps
// the row's cos/sin in registers for every (layer, head) slab it visits, and writes the
// de-rotated pairs to the workspace with the same layout as the source.
// ---------------------------------------------------------------------------------------

// The producer and the recode stream every element once: loads and stores carry the
// non-temporal hint (3-5 % faster on the headline de-rotation and recode than plain ones).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Vec16;  // 16 bytes of elements, widened to fp32

template <>
struct Vec16<true> {
    static constexpr int N = 8;
    uint4 raw;
    __device__ __forceinline__ void load(const void* p) {
        const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt*)p);
        raw = make_uint4(v[0], v[1], v[2], v[3]);
    }
    __device__ __forceinline__ float get(int v) const {
        const uint32_t w = (&raw.x)[v >> 1];
        return (v & 1) ? bf16hi(w) : bf16lo(w);
    }
    __device__ __forceinline__ static void store(void* p, const float* x) {
        uint4 o;
        o.x = pack_bf16(x[0], x[1]);
        o.y = pack_bf16(x[2], x[3]);
        o.z = pack_bf16(x[4], x[5]);
        o.w = pack_bf16(x[6], x[7]);
        const u32x4_nt v = {o.x, o.y, o.z, o.w};
        __builtin_nontemporal_store(v, (u32x4_nt*)p);
    }
};

template <>
struct Vec16<false> {
    static constexpr int N = 4;
    float4 raw;
    __device__ __forceinline__ void load(const void* p) {
        const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt*)p);
        raw = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
    }
    __device__ __forceinline__ float get(int v) const { return (&raw.x)[v]; }
    __device__ __forceinline__ static void store(void* p, const float* x) {
        const u32x4_nt v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
        __builtin_nontemporal_store(v, (u32x4_nt*)p);
    }
};

template <bool BF16, int D>
__global__ __launch_bounds__(256) void derope_kernel(const void* __restrict__ src,
                                                     void* __restrict__ ws,
                                                     const int32_t* __restrict__ layers,
                                                     int n_layers, int H, int64_t T,
                                                     const float2* __restrict__ tab) {
    using V = Vec16<BF16>;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int VEC = V::N;
    constexpr int HALF = D / 2;
    constexpr int TPR = HALF / VEC;  // threads per token row
    constexpr int RPB = 256 / TPR;   // token rows per block
    constexpr int UNROLL = 4;
    const int tid = threadIdx.x;
    const int q = tid % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
    if (row >= T) return;

    float c[VEC], s[VEC];
    {
        const float4* tr = (const float4*)(tab + row * HALF + q * VEC);
#pragma unroll
        for (int v = 0; v < VEC / 2; ++v) {
            const float4 cs = tr[v];
            c[2 * v] = cs.x; s[2 * v] = cs.y;
            c[2 * v + 1] = cs.z; s[2 * v + 1] = cs.w;
        }
    }
    const char* srcb = (const char*)src;
    char* wsb = (char*)ws;
    const int nslabs = n_layers * H;
    const int step = gridDim.y;
    for (int s0 = blockIdx.y; s0 < nslabs; s0 += step * UNROLL) {
        V lo[UNROLL], hi[UNROLL];
        size_t off[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int sl = s0 + u * step;
            off[u] = 0;
            if (sl < nslabs) {
                const int l = layers[sl / H];
                const int h = sl - (sl / H) * H;
                off[u] = ((((size_t)l * H + h) * (size_t)T + (size_t)row) * D + q * VEC) * ES;
                lo[u].load(srcb + off[u]);
                hi[u].load(srcb + off[u] + HALF * ES);
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (s0 + u * step < nslabs) {
                float ol[VEC], oh[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const float xl = lo[u].get(v), xh = hi[u].get(v);
                    ol[v] = fmaf(xh, s[v], xl * c[v]);   // rotate by -a
                    oh[v] = fmaf(-xl, s[v], xh * c[v]);
                }
                V::store(wsb + off[u], ol);
                V::store(wsb + off[u] + HALF * ES, oh);
            }
        }
    }
}

hipError_t launch_derope(Elem e, const void* src, void* ws, const int32_t* layers, int n_layers,
                         const ApplyGeom& g, const float2* tab, hipStream_t s) {
    const int vec = (e == Elem::BF16) ? 8 : 4;
    const int tpr = (g.d / 2) / vec;
    const int rpb = 256 / tpr;
    const int64_t bx = (g.T + rpb - 1) / rpb;
    const int nslabs = n_layers * g.H;
    int64_t by = (4096 + bx - 1) / bx;
    if (by > nslabs) by = nslabs;
    if (by < 1) by = 1;
    const dim3 grid((unsigned)bx, (unsigned)by);
#define KVMAP_DEROPE(B, D) \
    hipLaunchKernelGGL((derope_kernel<B, D>), grid, dim3(256), 0, s, src, ws, layers, n_layers, g.H, g.T, tab)
    if (e == Elem::BF16) {
        if (g.d == 128) KVMAP_DEROPE(true, 128); else KVMAP_DEROPE(true, 64);
    } else {
        if (g.d == 128) KVMAP_DEROPE(false, 128); else KVMAP_DEROPE(false, 64);
    }
#undef KVMAP_DEROPE
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Rows for the fit-side statistics: out[t][(j*H + h)*d + e] = layer layers[j], head h, token t,
// element e of a cache [L][H][T][d], optionally with its RoPE stripped (the content space in
// which the maps are fitted, VeloxQuant-MLX "Cross-Model KV Transfer", "The mapping": keys are
// de-rotated with each model's own rotation before any statistics).  Same thread layout as the
// producer above; each (layer, head) slab of a token row lands as d contiguous elements of
// the output row.
// ---------------------------------------------------------------------------------------

template <bool BF16, int D, bool STRIP>
__global__ __launch_bounds__(256) void rows_kernel(const void* __restrict__ src, void* __restrict__ out,
                                                   RowLayers layers, int n_layers, int H, int64_t T,
                                                   const float2* __restrict__ tab) {
    using V = Vec16<BF16>;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int VEC = V::N;
    constexpr int HALF = D / 2;
    constexpr int TPR = HALF / VEC;
    constexpr int RPB = 256 / TPR;
    const int tid = threadIdx.x;
    const int q = tid % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
    if (row >= T) return;
    float c[VEC], s[VEC];
    if (STRIP) {
        const float4* tr = (const float4*)(tab + row * HALF + q * VEC);
#pragma unroll
        for (int v = 0; v < VEC / 2; ++v) {
            const float4 cs = tr[v];
            c[2 * v] = cs.x; s[2 * v] = cs.y;
            c[2 * v + 1] = cs.z; s[2 * v + 1] = cs.w;
        }
    }
    const char* srcb = (const char*)src;
    char* outb = (char*)out;
    const int nslabs = n_layers * H;
    for (int sl = blockIdx.y; sl < nslabs; sl += gridDim.y) {
        const int j = sl / H, h = sl - (sl / H) * H;
        const size_t in_off = ((((size_t)layers.l[j] * H + h) * (size_t)T + (size_t)row) * D + q * VEC) * ES;
        const size_t out_off = (((size_t)row * nslabs + sl) * D + q * VEC) * ES;
        V lo, hi;
        lo.load(srcb + in_off);
        hi.load(srcb + in_off + HALF * ES);
        float ol[VEC], oh[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float xl = lo.get(v), xh = hi.get(v);
            if (STRIP) {
                ol[v] = fmaf(xh, s[v], xl * c[v]);  // rotate by -a
                oh[v] = fmaf(-xl, s[v], xh * c[v]);
            } else {
                ol[v] = xl;
                oh[v] = xh;
            }
        }
        V::store(outb + out_off, ol);
        V::store(outb + out_off + HALF * ES, oh);
    }
}

hipError_t launch_rows(Elem e, const void* src, void* out, const RowLayers& layers, int n_layers, int H,
                       int64_t T, int d, const float2* tab, hipStream_t s) {
    const int vec = (e == Elem::BF16) ? 8 : 4;
    const int rpb = 256 / ((d / 2) / vec);
    const int64_t bx = (T + rpb - 1) / rpb;
    const int nslabs = n_layers * H;
    int64_t by = (4096 + bx - 1) / bx;
    if (by > nslabs) by = nslabs;
    if (by < 1) by = 1;
    const dim3 grid((unsigned)bx, (unsigned)by);
#define KVMAP_ROWS(B, D, S) \
    hipLaunchKernelGGL((rows_kernel<B, D, S>), grid, dim3(256), 0, s, src, out, layers, n_layers, H, T, tab)
    const bool strip = tab != nullptr;
    if (e == Elem::BF16) {
        if (d == 128) { if (strip) KVMAP_ROWS(true, 128, true); else KVMAP_ROWS(true, 128, false); }
        else { if (strip) KVMAP_ROWS(true, 64, true); else KVMAP_ROWS(true, 64, false); }
    } else {
        if (d == 128) { if (strip) KVMAP_ROWS(false, 128, true); else KVMAP_ROWS(false, 128, false); }
        else { if (strip) KVMAP_ROWS(false, 64, true); else KVMAP_ROWS(false, 64, false); }
    }
#undef KVMAP_ROWS
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Non-finite scan (optional guard: reject NaN/Inf mapped caches rather than pass them on,
// as the KVBridge README's "Failure is a first-class outcome" section asks of a guarded
// transfer).
// ---------------------------------------------------------------------------------------

template <bool BF16>
__global__ __launch_bounds__(256) void count_nonfinite_kernel(const void* __restrict__ p,
                                                              int64_t n,
                                                              unsigned int* __restrict__ count) {
    unsigned int local = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (BF16) {
            const uint16_t u = ((const uint16_t*)p)[i];
            local += ((u & 0x7F80u) == 0x7F80u);
        } else {
            const uint32_t u = ((const uint32_t*)p)[i];
            local += ((u & 0x7F800000u) == 0x7F800000u);
        }
    }
    if (local) atomicAdd(count, local);
}

hipError_t launch_count_nonfinite(Elem e, const void* p, int64_t n, unsigned int* count,
                                  hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (e == Elem::BF16)
        hipLaunchKernelGGL(count_nonfinite_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, count);
    else
        hipLaunchKernelGGL(count_nonfinite_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, count);
    return hipGetLastError();
}

}  // namespace kvmap
