// The map GEMM for short caches (T up to a few hundred tokens), bf16.  At these lengths the
// apply moves the whole of W (F x N per target layer, K and V) for little arithmetic, so it
// is bound by reading W from HBM (VeloxQuant-MLX "Cross-Model KV Transfer", "The mapping":
// one ridge map per target head; the same Y = X W + b, then bias and target RoPE).  The
// long-cache kernel's 256-token tiles would be mostly padding here and would leave only a
// few hundred workgroups to stream W, so this path
//   * tiles 256 features x 64 tokens, and splits the reduction over KS groups of K-steps,
//     so that enough workgroups stream disjoint parts of W (about 4096 for caches of up to
//     16 tokens; longer ones do not split, the partial sums would cost more than they gain);
//   * writes each split's fp32 partial sums, and a second kernel adds them in a fixed order
//     (deterministic), adds the bias and applies the target RoPE (keys), rounding once to
//     bf16 into the target cache layout [t][h][p][e].
// The gather is the long-cache kernel's: one K-step of 64 features lies in one (selected
// layer, source head) slab, so a K-step only moves the slab's base address.

#include <algorithm>

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

namespace kvmap {

namespace {

constexpr int SBM = 256;                          // features per tile
constexpr int SBN = 64;                           // tokens per tile
constexpr int SBK = 64;                           // features (reduction) per K-step
constexpr int NRING = 4;                          // stages in flight + the one computed
constexpr int W_CHUNKS = SBM * SBK / 8;           // 16-byte chunks of W per stage (2048)
constexpr int X_CHUNKS = SBN * SBK / 8;           // ... of X (512)
constexpr int STAGE = (W_CHUNKS + X_CHUNKS) * 16;  // 40 KB
constexpr int LW = W_CHUNKS / 512, LX = X_CHUNKS / 512;  // loads per thread per stage (4, 1)
constexpr int LPS = LW + LX;

}  // namespace

// Workgroup b: split ks = b % KS, then feature tile, token tile, (t, K|V).  8 waves: wave w
// computes features (w & 1) * 128 .. + 127 (whole heads) of tokens (w >> 1) * 16 .. + 15,
// as 8 blocks of v_mfma_f32_16x16x32_bf16.  Ring of 4 stages (W tile + X tile), each filled
// by buffer_load_dwordx4 ... lds three K-steps ahead of its use.
template <int D>
__global__ __launch_bounds__(512) void map_bf16_small_kernel(MapArgs a, int L_tgt, int H, int k, int64_t T,
                                                             int nN, int nP, int KS, int kps,
                                                             float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) char smem[NRING * STAGE];
    uint4* lds = (uint4*)smem;

    int b = blockIdx.x;
    const int ks = b % KS;
    b /= KS;
    const int nb = b % nN;
    b /= nN;
    const int pb = b % nP;
    b /= nP;
    const int kv = b & 1, t = b >> 1;
    if (t >= L_tgt) return;

    const int N = H * D, F = k * N;
    const int nk_all = F / SBK;
    const int kt0 = ks * kps;
    const int nk = min(kps, nk_all - kt0);  // >= 1 (the host sizes KS so)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = nb * SBM, p0 = pb * SBN;
    const uint16_t* __restrict__ X = (const uint16_t*)(kv ? a.xv : a.xk);
    const uint16_t* __restrict__ W = (const uint16_t*)(kv ? a.Wv : a.Wk) + (size_t)t * N * F;
    const size_t slab = (size_t)T * D;
    const uint32_t slab_bytes = (uint32_t)(slab * 2);
    const uint64_t lbase = (uint64_t)(uintptr_t)(X + (size_t)(lane < k ? a.sel[t * k + lane] : 0) * H * slab);
    const int lb_lo = (int)(uint32_t)lbase, lb_hi = (int)(uint32_t)(lbase >> 32);
    const i32x4_t wr = make_rsrc(W, (uint32_t)((size_t)N * F * 2));
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);

    // Loads: W slot u = i*512 + tid holds row u/8, chunk (u%8) ^ slot_xor(row); X slot tid
    // holds row tid/8 likewise.  Rows past N or T repeat the last one (never stored).
    int aoff[LW], boff;
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int r = i * 64 + wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        aoff[i] = (min(n0 + r, N - 1) * F + c * 8) * 2;
    }
    {
        const int r = wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        boff = ((int)(min((int64_t)(p0 + r), T - 1) * D) + c * 8) * 2;
    }
    // Issue state: W byte offset of the next K-step; gathered slab (head h of selected layer
    // j) and feature offset in its rows; all stop at the split's last K-step (the extra
    // stages the pipeline loads at the end repeat it and are never read).
    const int w_last = (kt0 + nk - 1) * SBK * 2;
    int w_soff = kt0 * SBK * 2;
    const int per = H * D;
    // (divisions by the runtime H*D are vector code: read the uniform results back into SGPRs)
    int x_j = __builtin_amdgcn_readfirstlane((kt0 * SBK) / per);
    int x_h = __builtin_amdgcn_readfirstlane(((kt0 * SBK) % per) / D);
    int x_eb = __builtin_amdgcn_readfirstlane(((kt0 * SBK) % D) * 2);
    int x_left = nk;  // K-steps of the split not yet issued
    const uint64_t x0 = (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(lb_hi, x_j) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane(lb_lo, x_j)) +
                        (uint64_t)x_h * slab_bytes;
    uint32_t x_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x0);
    uint32_t x_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x0 >> 32));
    int s_buf = 0;
    auto issue = [&]() {
        const uint32_t la = lds_base + (uint32_t)s_buf * STAGE + wave_s * 1024u;
        const i32x4_t xr = {(int)x_lo, (int)x_hi, (int)slab_bytes, 0x00020000};
#pragma unroll
        for (int i = 0; i < LW; ++i) lds_dma16(wr, la + i * 8192u, aoff[i], w_soff);
        lds_dma16(xr, la + (uint32_t)(W_CHUNKS * 16), boff, x_eb);
        s_buf = (s_buf + 1 == NRING) ? 0 : s_buf + 1;
        // advance (held at the split's last K-step once it has been issued)
        const int adv = x_left > 1;
        x_left -= adv;
        w_soff = min(w_soff + adv * SBK * 2, w_last);
        const int eb = x_eb + adv * SBK * 2;
        const int we = (eb == D * 2);
        x_eb = we ? 0 : eb;
        const int hh = x_h + we;
        const int wh = (hh == H);
        x_h = wh ? 0 : hh;
        x_j = min(x_j + wh, k - 1);
        const uint32_t a_lo = x_lo + (we ? slab_bytes : 0u);
        const uint32_t a_hi = x_hi + (a_lo < x_lo ? 1u : 0u);
        x_lo = uniform_select(wh, (uint32_t)__builtin_amdgcn_readlane(lb_lo, x_j), a_lo);
        x_hi = uniform_select(wh, (uint32_t)__builtin_amdgcn_readlane(lb_hi, x_j), a_hi);
    };

    constexpr int IB = 8;
    f32x4_t acc[IB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;
    const int wn = wave & 1, wp = wave >> 1;
    const int kq = lane >> 4;
    const int fx = slot_xor(lane & 15);
    const int arow = (wn * 128 + (lane & 15)) * 8;
    const int brow = W_CHUNKS + (wp * 16 + (lane & 15)) * 8;

#pragma unroll
    for (int s = 0; s < NRING; ++s) issue();
    wait_vmcnt<(NRING - 1) * LPS>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int kk = 0; kk < nk; ++kk) {
        const uint4* st = lds + (kk % NRING) * (STAGE / 16);
        bf16x8_t fa[2][IB], fb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int slot = (h * 4 + kq) ^ fx;
#pragma unroll
            for (int i = 0; i < IB; ++i) fa[h][i] = __builtin_bit_cast(bf16x8_t, st[arow + i * 128 + slot]);
            fb[h] = __builtin_bit_cast(bf16x8_t, st[brow + slot]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < IB; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[h][i], fb[h], acc[i], 0, 0, 0);
        // every read of stage kk returned, stage kk+1 landed (kk+2 and kk+3 may be in flight);
        // after the barrier its buffer takes stage kk+4
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<(NRING - 2) * LPS>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue();
    }
    wait_vmcnt<0>();

    // partial sums: lane holds features 4 (lane / 16) + r of each 16 x 16 block, token lane % 16
    const int p = p0 + wp * 16 + (lane & 15);
    if (p < T) {
        float* dst = part + ((((size_t)ks * L_tgt + t) * 2 + kv) * (size_t)T + p) * N;
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            const int n = n0 + wn * 128 + i * 16 + kq * 4;
            if (n < N) *(float4*)(dst + n) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        }
    }
}

// Sum of the KS partials in split order, + bias, target RoPE on keys, bf16 into [t][h][p][e].
// Thread: 4 RoPE pairs (e .. e+3, e+d/2 .. e+d/2+3) of one head of one token.
template <int D>
__global__ __launch_bounds__(256) void map_small_reduce_kernel(MapArgs a, const float* __restrict__ part, int L_tgt,
                                                               int H, int64_t T, int KS) {
    constexpr int HALF = D / 2, QG = HALF / 4;
    const int N = H * D;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)L_tgt * 2 * T * H * QG;
    if (idx >= total) return;
    int64_t r = idx;
    const int q = (int)(r % QG);
    r /= QG;
    const int h = (int)(r % H);
    r /= H;
    const int64_t p = r % T;
    r /= T;
    const int kv = (int)(r & 1), t = (int)(r >> 1);
    const int e = q * 4, nlo = h * D + e;
    float lo[4] = {0.f, 0.f, 0.f, 0.f}, hi[4] = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
        const float* src = part + ((((size_t)ks * L_tgt + t) * 2 + kv) * (size_t)T + p) * N;
        const float4 l4 = *(const float4*)(src + nlo), h4 = *(const float4*)(src + nlo + HALF);
        lo[0] += l4.x; lo[1] += l4.y; lo[2] += l4.z; lo[3] += l4.w;
        hi[0] += h4.x; hi[1] += h4.y; hi[2] += h4.z; hi[3] += h4.w;
    }
    const uint16_t* __restrict__ bias = (const uint16_t*)(kv ? a.bv : a.bk) + (size_t)t * N;
    const uint2 bl = *(const uint2*)(bias + nlo), bh = *(const uint2*)(bias + nlo + HALF);
    lo[0] += bf16lo(bl.x); lo[1] += bf16hi(bl.x); lo[2] += bf16lo(bl.y); lo[3] += bf16hi(bl.y);
    hi[0] += bf16lo(bh.x); hi[1] += bf16hi(bh.x); hi[2] += bf16lo(bh.y); hi[3] += bf16hi(bh.y);
    if (kv == 0) {
        const float4* cs4 = (const float4*)(a.tab_tgt + p * HALF + e);
        const float4 c01 = cs4[0], c23 = cs4[1];
        const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
        const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float l = lo[v], hh = hi[v];
            lo[v] = fmaf(-hh, ss[v], l * cc[v]);
            hi[v] = fmaf(l, ss[v], hh * cc[v]);
        }
    }
    uint16_t* out = (uint16_t*)(kv ? a.outv : a.outk) + ((((size_t)t * H + h) * T + p) * D);
    *(uint2*)(out + e) = make_uint2(pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]));
    *(uint2*)(out + e + HALF) = make_uint2(pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3]));
}

// ---------------------------------------------------------------------------------------

SmallPlan map_bf16_small_plan(const ApplyGeom& g) {
    SmallPlan pl;
    pl.nN = (g.N() + SBM - 1) / SBM;
    pl.nP = (int)((g.T + SBN - 1) / SBN);
    const int nk_all = g.F() / SBK;
    const int tiles = g.L_tgt * 2 * pl.nN * pl.nP;
    // Splits trade parallel W streams against the partial sums' traffic (KS x T x N fp32 per
    // target layer and K/V, written and read back by the reduce).  Measured at the 14B->32B maps
    // (512 tiles): about 4096 workgroups are best up to 16 tokens (0.394 ms at T = 1 against
    // 0.430 with 2048), about 512 -- no split -- from 32 on (0.493 ms at T = 64 against 0.538).
    const int target = g.T <= 16 ? 4096 : 512;
    int ks = (target + tiles - 1) / tiles;
    ks = std::max(1, std::min(ks, nk_all));
    pl.kps = (nk_all + ks - 1) / ks;
    pl.KS = (nk_all + pl.kps - 1) / pl.kps;  // every split non-empty
    pl.part_bytes = (size_t)pl.KS * g.L_tgt * 2 * (size_t)g.T * g.N() * sizeof(float);
    return pl;
}

hipError_t launch_map_bf16_small(const MapArgs& a, const ApplyGeom& g, const SmallPlan& pl, float* part,
                                 hipStream_t s) {
    const unsigned blocks = (unsigned)(g.L_tgt * 2 * pl.nN * pl.nP * pl.KS);
    const int64_t rthreads = (int64_t)g.L_tgt * 2 * g.T * g.H * (g.d / 8);
    const unsigned rblocks = (unsigned)((rthreads + 255) / 256);
    if (g.d == 128) {
        hipLaunchKernelGGL((map_bf16_small_kernel<128>), dim3(blocks), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T,
                           pl.nN, pl.nP, pl.KS, pl.kps, part);
        hipLaunchKernelGGL((map_small_reduce_kernel<128>), dim3(rblocks), dim3(256), 0, s, a, part, g.L_tgt, g.H,
                           g.T, pl.KS);
    } else {
        hipLaunchKernelGGL((map_bf16_small_kernel<64>), dim3(blocks), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T,
                           pl.nN, pl.nP, pl.KS, pl.kps, part);
        hipLaunchKernelGGL((map_small_reduce_kernel<64>), dim3(rblocks), dim3(256), 0, s, a, part, g.L_tgt, g.H,
                           g.T, pl.KS);
    }
    return hipGetLastError();
}

}  // namespace kvmap
