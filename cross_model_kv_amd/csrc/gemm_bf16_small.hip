// The map GEMM for short caches (up to 128 tokens), bf16.  At these lengths the apply moves the
// whole of W (F x N per target layer, K and V) for little arithmetic, so it is bound by reading
// W from HBM (VeloxQuant-MLX "Cross-Model KV Transfer", "The mapping": one ridge map per target
// head; the same Y = X W + b, then bias and target RoPE).  The long-cache kernel's 256-token
// tiles would be mostly padding here and its one-tile workgroups would drain and refill their
// load pipeline per tile, so this path
//   * tiles 256 features x 16, 32, 64 or 128 tokens and runs one persistent workgroup per compute
//     unit; each streams its share of the work items (a tile, or a split of a tile's K
//     reduction when the tiles do not divide evenly over the compute units) through one ring
//     of LDS stages that runs on from item to item;
//   * loads W, which is read exactly once, with the non-temporal hint (7.2 against 5.9 TB/s
//     for a plain stream on gfx950);
//   * writes each item's fp32 partial sums, and a second kernel adds them in a fixed order
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

constexpr int SBM = 256;                 // features per tile
constexpr int SBN = 128;                 // most tokens per tile (the path takes T <= SBN)
constexpr int SBK = 64;                  // features (reduction) per K-step
constexpr int W_CHUNKS = SBM * SBK / 8;  // 16-byte chunks of W per stage (2048)
constexpr int LW = W_CHUNKS / 512;       // W loads per thread per stage (4)

#ifndef KVMAP_SMALL_NT
#define KVMAP_SMALL_NT true
#endif

}  // namespace

// Work item i of n_items = tiles x KS: split i % KS (K-steps kt0 .. kt0 + nk - 1) of feature
// tile (i / KS) % nN of target layer (i / (KS nN)) % L_tgt, keys for the first L_tgt KS nN
// items, values after them.  Uniform scalars.  The items in flight at one time (consecutive
// indices) thus read one contiguous span of one map tensor: interleaving the K and V maps,
// two allocations about a gigabyte apart read at the same offsets in lockstep, measured 25 %
// slower at the 14B->32B maps.
struct ShortItem {
    int t, kv, n0, ks, kt0, nk;
};

__device__ __forceinline__ ShortItem short_item(int i, int KS, int nN, int L_tgt, int kps, int nk_all) {
    ShortItem it;
    it.ks = i % KS;
    i /= KS;
    it.n0 = (i % nN) * SBM;
    i /= nN;
    it.t = i % L_tgt;
    it.kv = i / L_tgt;
    it.kt0 = it.ks * kps;
    it.nk = min(kps, nk_all - it.kt0);
    return it;
}

// Items finish inside the short-cache kernel (bias, target RoPE, bf16 output; no reduce kernel)
// when the K reduction is not split and a tile holds 64 or 128 tokens.  The host and the kernel
// both decide by this.
__host__ __device__ __forceinline__ bool small_fused(int tok, int KS) { return tok >= 64 && KS == 1; }

// Persistent: workgroup g (one per compute unit) takes items g, g + G, g + 2G, ... and streams
// them through ONE ring of NRING stages (W tile + X tile), each filled by buffer_load_dwordx4
// ... lds NRING - 1 K-steps ahead of its use.  The ring runs on across items: the loads of an
// item's first K-steps go out while the previous item's last ones are computed, so W streams
// without a drain and refill per tile.  At the end of an item its fp32 partial sums are stored
// (or, with an unsplit K reduction at 64 or 128 tokens, its finished bf16 rows) and the
// accumulators cleared.  TOK (16, 32, 64 or 128, at least T) tokens per tile, 8 waves:
// WN waves side by side along the features, each FW features (whole 16-feature blocks) x TW
// tokens as IB x JB blocks of v_mfma_f32_16x16x32_bf16 -- 8 x 1 waves of 32 x 16 at TOK 16,
// 4 x 2 of 64 x 16 at 32, 2 x 4 of 128 x 16 at 64, 2 x 4 of 128 x 32 at 128 -- so that short
// caches spend no MFMAs and fragment reads on padding tokens.  The ring has 4 stages (34 to 40
// KB) up to 64 tokens and 3 (48 KB) at 128.  NT: W (read exactly once) is loaded with the
// non-temporal hint.
template <int D, int TOK, bool NT>
__global__ __launch_bounds__(512) void map_bf16_small_kernel(MapArgs a, int L_tgt, int H, int k, int64_t T,
                                                             int nN, int KS, int kps, int n_items,
                                                             float* __restrict__ part) {
    static_assert(TOK == 16 || TOK == 32 || TOK == 64 || TOK == 128, "tokens per tile");
    constexpr int X_CHUNKS = TOK * SBK / 8;            // 16-byte chunks of X per stage
    constexpr int LX = X_CHUNKS > 512 ? X_CHUNKS / 512 : 1;  // X loads per loading lane
    constexpr int XW = X_CHUNKS / (64 * LX);           // waves that load X
    constexpr int STAGE = (W_CHUNKS + X_CHUNKS) * 16;  // 34, 36, 40 or 48 KB
    constexpr int NRING = TOK == 128 ? 3 : 4;          // stages in the ring (LDS: 136 - 160 KB)
    constexpr int WN = TOK <= 64 ? 128 / TOK : 2;      // waves along the features
    constexpr int TW = TOK / (8 / WN);                 // tokens per wave
    constexpr int FW = SBM / WN;                       // features per wave
    constexpr int IB = FW / 16;                        // 16-feature MFMA blocks per wave
    constexpr int JB = TW / 16;                        // 16-token MFMA blocks per wave
    __shared__ __attribute__((aligned(16))) char smem[NRING * STAGE];
    const uint4* lds = (const uint4*)smem;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    if (g >= n_items) return;  // (the host launches at most n_items workgroups)

    const int N = H * D, F = k * N;
    const int nk_all = F / SBK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t slab = (size_t)T * D;
    const uint32_t slab_bytes = (uint32_t)(slab * 2);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);

    // Loads: W slot u = i*512 + tid holds row u/8, chunk (u%8) ^ slot_xor(row); X slot u =
    // i*512 + tid (u < X_CHUNKS) holds row u/8 likewise.  Rows past N or T repeat the last one
    // (never stored).
    int arow[LW], acol[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        arow[i] = i * 64 + wave * 8 + (lane >> 3);
        acol[i] = ((lane & 7) ^ slot_xor(arow[i])) * 8;
    }
    int boff[LX];
#pragma unroll
    for (int i = 0; i < LX; ++i) {
        const int r = i * 64 + wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        boff[i] = (int)(((uint32_t)min((int64_t)r, T - 1) * (uint32_t)D + (uint32_t)c * 8u) * 2u);
    }

    // ---- issue side: the item whose stages are being loaded, and its position ----
    // W: descriptor of W[t] (K or V), per-lane row offsets, byte offset of the next K-step.
    // X: the gathered slab (head x_h of selected layer x_j) and the K-step's byte offset in
    // its rows.  x_left = K-steps of the item not yet issued; past the last K-step of the
    // last item the issue repeats that K-step (in bounds, never read).
    int is_item = g, is_t = 0, x_left = 0, x_j = 0, x_h = 0, x_eb = 0, w_soff = 0;
    int aoff[LW];
    i32x4_t wr;
    const uint16_t* is_x = nullptr;  // K or V cache (de-rotated keys or values)
    uint64_t x_addr = 0;             // address of the current slab
    auto x_slab = [&](int j, int h) {
        const int layer = scalar_load_dword(a.sel + is_t * k + j);
        return (uint64_t)(uintptr_t)is_x + ((uint64_t)layer * H + h) * slab_bytes;
    };
    auto begin_item = [&](int item) {
        const ShortItem it = short_item(item, KS, nN, L_tgt, kps, nk_all);
        is_t = __builtin_amdgcn_readfirstlane(it.t);
        const int kv = __builtin_amdgcn_readfirstlane(it.kv);
        const int n0 = __builtin_amdgcn_readfirstlane(it.n0);
        const int kt0 = __builtin_amdgcn_readfirstlane(it.kt0);
        const uint16_t* W = (const uint16_t*)(kv ? a.Wv : a.Wk) + (size_t)is_t * N * F;
        wr = make_rsrc(W, (uint32_t)((size_t)N * F * 2));
        is_x = (const uint16_t*)(kv ? a.xv : a.xk);
#pragma unroll
        for (int i = 0; i < LW; ++i)  // byte offsets below 2^32 (N F < 2^31 is validated)
            aoff[i] = (int)(((uint32_t)min(n0 + arow[i], N - 1) * (uint32_t)F + (uint32_t)acol[i]) * 2u);
        w_soff = kt0 * SBK * 2;
        const int f0 = kt0 * SBK, per = H * D;
        x_j = __builtin_amdgcn_readfirstlane(f0 / per);
        x_h = __builtin_amdgcn_readfirstlane((f0 % per) / D);
        x_eb = __builtin_amdgcn_readfirstlane((f0 % D) * 2);
        x_left = __builtin_amdgcn_readfirstlane(it.nk);
        x_addr = x_slab(x_j, x_h);
    };
    int s_buf = 0;
    auto issue = [&]() {
        const uint32_t la = lds_base + (uint32_t)s_buf * STAGE + wave_s * 1024u;
        const i32x4_t xr = {(int)(uint32_t)x_addr, (int)(uint32_t)(x_addr >> 32), (int)slab_bytes, 0x00020000};
#pragma unroll
        for (int i = 0; i < LW; ++i) {
            if constexpr (NT)
                lds_dma16_nt(wr, la + i * 8192u, aoff[i], w_soff);
            else
                lds_dma16(wr, la + i * 8192u, aoff[i], w_soff);
        }
        if (wave_s < XW) {
#pragma unroll
            for (int i = 0; i < LX; ++i) lds_dma16(xr, la + (uint32_t)(W_CHUNKS * 16) + i * 8192u, boff[i], x_eb);
        }
        s_buf = (s_buf + 1 == NRING) ? 0 : s_buf + 1;
        if (x_left > 1) {  // next K-step of the item
            --x_left;
            w_soff += SBK * 2;
            x_eb += SBK * 2;
            if (x_eb == D * 2) {  // next head
                x_eb = 0;
                if (++x_h == H) {  // next selected layer
                    x_h = 0;
                    ++x_j;
                    x_addr = x_slab(x_j, 0);
                } else {
                    x_addr += slab_bytes;
                }
            }
        } else if (is_item + G < n_items) {  // first K-step of the next item
            is_item += G;
            begin_item(is_item);
        }
    };

    f32x4_t acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
    const int wn = wave % WN, wp = wave / WN;
    const int kq = lane >> 4;

    // End of an item, split K reduction: its fp32 partial sums, summed by the reduce kernel.
    auto store_partial = [&](const ShortItem& it) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int p = wp * TW + j * 16 + (lane & 15);
            if (p >= T) continue;
            float* dst = part + ((((size_t)it.ks * L_tgt + it.t) * 2 + it.kv) * (size_t)T + p) * N;
#pragma unroll
            for (int i = 0; i < IB; ++i) {
                const int n = it.n0 + wn * FW + i * 16 + kq * 4;
                if (n < N)
                    *(float4*)(dst + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    };
    // End of an item, whole K reduction at 64 or 128 tokens per tile: a wave's 128 features are
    // whole heads, so both members (e, e + d/2) of every RoPE pair sit in one lane (blocks i and
    // i + d/32) and the item finishes here as the reduce kernel would finish it (+ bias, target
    // RoPE on keys, bf16 into [t][h][p][e]; the same fp32 operations, so the same bits).
    auto finish_item = [&](const ShortItem& it) {
        if constexpr (TOK >= 64) {
            constexpr int HALF = D / 2, PB = HALF / 16, NLO = IB / 2;
            static_assert(FW % D == 0, "a wave's features are whole heads");
            const uint16_t* __restrict__ bias = (const uint16_t*)(it.kv ? a.bv : a.bk) + (size_t)it.t * N;
            uint16_t* __restrict__ out = (uint16_t*)(it.kv ? a.outv : a.outk);
#pragma unroll
            for (int li = 0; li < NLO; ++li) {
                const int i = (li / PB) * 2 * PB + li % PB;         // block of low members
                const int nl = it.n0 + wn * FW + i * 16 + kq * 4;  // the lane's first low member
                if (nl >= N) continue;  // a head past the last one (partial last feature tile)
                const int h = nl / D, e = nl - h * D;
                const uint2 bl = *(const uint2*)(bias + nl), bh = *(const uint2*)(bias + nl + HALF);
                const float bL[4] = {bf16lo(bl.x), bf16hi(bl.x), bf16lo(bl.y), bf16hi(bl.y)};
                const float bH[4] = {bf16lo(bh.x), bf16hi(bh.x), bf16lo(bh.y), bf16hi(bh.y)};
#pragma unroll
                for (int j = 0; j < JB; ++j) {
                    const int64_t p = wp * TW + j * 16 + (lane & 15);
                    if (p >= T) continue;
                    float lo[4], hi[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        lo[r] = (0.f + acc[i][j][r]) + bL[r];
                        hi[r] = (0.f + acc[i + PB][j][r]) + bH[r];
                    }
                    if (it.kv == 0) {
                        const float4* cs4 = (const float4*)(a.tab_tgt + p * HALF + e);
                        const float4 c01 = cs4[0], c23 = cs4[1];
                        const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
                        const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float l = lo[r], hh = hi[r];
                            lo[r] = fmaf(-hh, ss[r], l * cc[r]);
                            hi[r] = fmaf(l, ss[r], hh * cc[r]);
                        }
                    }
                    uint16_t* dst = out + (((size_t)it.t * H + h) * T + p) * D + e;
                    *(uint2*)dst = make_uint2(pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]));
                    *(uint2*)(dst + HALF) = make_uint2(pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3]));
                }
            }
        }
    };
    const int fx = slot_xor(lane & 15);
    const int arow0 = (wn * FW + (lane & 15)) * 8;
    const int brow0 = W_CHUNKS + (wp * TW + (lane & 15)) * 8;

    begin_item(g);
#pragma unroll
    for (int s = 0; s < NRING; ++s) issue();
    // this wave's loads per stage: LW, plus LX X loads in the first XW waves
    if (wave_s < XW)
        wait_vmcnt<(NRING - 1) * (LW + LX)>();
    else
        wait_vmcnt<(NRING - 1) * LW>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    int c_item = g;                                                       // item being computed
    int c_left = short_item(g, KS, nN, L_tgt, kps, nk_all).nk;                   // its K-steps left
    int c_buf = 0;
    for (;;) {
        const uint4* st = lds + c_buf * (STAGE / 16);
        bf16x8_t fa[2][IB], fb[2][JB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int slot = (h * 4 + kq) ^ fx;
#pragma unroll
            for (int i = 0; i < IB; ++i) fa[h][i] = __builtin_bit_cast(bf16x8_t, st[arow0 + i * 128 + slot]);
#pragma unroll
            for (int j = 0; j < JB; ++j) fb[h][j] = __builtin_bit_cast(bf16x8_t, st[brow0 + j * 128 + slot]);
        }
        // all fragment reads in flight before the first MFMA waits for one
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[h][i], fb[h][j], acc[i][j], 0, 0, 0);
        // every read of this stage returned, the next one landed (the two after it may be in
        // flight); after the barrier this buffer takes the stage three K-steps ahead.  Vector
        // stores of an item's partial sums below only add younger operations to the count, so
        // they can only make this wait stricter, never let it pass early.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (wave_s < XW)
            wait_vmcnt<(NRING - 2) * (LW + LX)>();
        else
            wait_vmcnt<(NRING - 2) * LW>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue();
        c_buf = (c_buf + 1 == NRING) ? 0 : c_buf + 1;
        if (--c_left == 0) {
            // lane holds features 4 (lane / 16) + r of each 16 x 16 block, token lane % 16
            const ShortItem it = short_item(c_item, KS, nN, L_tgt, kps, nk_all);
            if (small_fused(TOK, KS))
                finish_item(it);
            else
                store_partial(it);
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
            c_item += G;
            if (c_item >= n_items) break;
            c_left = short_item(c_item, KS, nN, L_tgt, kps, nk_all).nk;
        }
    }
    wait_vmcnt<0>();  // the repeated tail stages must land before the workgroup's LDS is released
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

// Tokens per tile: the smallest of 16, 32, 64 and 128 that holds the cache.
static int small_tok(int64_t T) { return T <= 16 ? 16 : T <= 32 ? 32 : T <= 64 ? 64 : 128; }

SmallPlan map_bf16_small_plan(const ApplyGeom& g, int cus) {
    SmallPlan pl;
    pl.nN = (g.N() + SBM - 1) / SBM;
    pl.nP = (int)((g.T + SBN - 1) / SBN);  // 1: the path takes T <= SBN
    // validated shapes have F = k H d >= 64, so at least one K-step; the guard keeps the
    // split arithmetic below free of a division by zero for any other input
    const int nk_all = std::max(1, g.F() / SBK);
    const int tiles = g.L_tgt * 2 * pl.nN * pl.nP;
    cus = std::max(1, cus);
    // The persistent kernel needs no split for parallelism; a split only evens out the work
    // when the tiles do not divide over the compute units.  Take the split count that
    // minimises the K-steps of the busiest workgroup (fewest splits on a tie: every split
    // adds T x N fp32 partial sums per tile).
    int best = 1;
    int64_t best_steps = -1;
    for (int ks = 1; ks <= std::min(16, nk_all); ++ks) {
        const int kps = (nk_all + ks - 1) / ks;
        const int KS = (nk_all + kps - 1) / kps;
        const int64_t items = (int64_t)tiles * KS;
        const int64_t grid = std::min<int64_t>(items, cus);
        const int64_t steps = (items + grid - 1) / grid * kps;
        if (best_steps < 0 || steps < best_steps) {
            best_steps = steps;
            best = ks;
        }
    }
    pl.kps = (nk_all + best - 1) / best;
    pl.KS = (nk_all + pl.kps - 1) / pl.kps;  // every split non-empty
    pl.n_items = tiles * pl.KS;
    pl.grid = std::min(pl.n_items, cus);
    pl.fused = small_fused(small_tok(g.T), pl.KS);
    pl.part_bytes = pl.fused ? 0 : (size_t)pl.KS * g.L_tgt * 2 * (size_t)g.T * g.N() * sizeof(float);
    return pl;
}

template <int D, int TOK>
static void launch_short(const MapArgs& a, const ApplyGeom& g, const SmallPlan& pl, float* part, hipStream_t s) {
    hipLaunchKernelGGL((map_bf16_small_kernel<D, TOK, KVMAP_SMALL_NT>), dim3(pl.grid), dim3(512), 0, s, a, g.L_tgt,
                       g.H, g.k, g.T, pl.nN, pl.KS, pl.kps, pl.n_items, part);
}

template <int D>
static void launch_short_d(const MapArgs& a, const ApplyGeom& g, const SmallPlan& pl, float* part, hipStream_t s) {
    switch (small_tok(g.T)) {
        case 16: launch_short<D, 16>(a, g, pl, part, s); break;
        case 32: launch_short<D, 32>(a, g, pl, part, s); break;
        case 64: launch_short<D, 64>(a, g, pl, part, s); break;
        default: launch_short<D, 128>(a, g, pl, part, s); break;
    }
}

hipError_t launch_map_bf16_small(const MapArgs& a, const ApplyGeom& g, const SmallPlan& pl, float* part,
                                 hipStream_t s) {
    if (g.T < 1 || g.T > SBN) return hipErrorInvalidValue;
    const int64_t rthreads = (int64_t)g.L_tgt * 2 * g.T * g.H * (g.d / 8);
    const unsigned rblocks = (unsigned)((rthreads + 255) / 256);
    if (pl.fused != small_fused(small_tok(g.T), pl.KS)) return hipErrorInvalidValue;  // a plan of another shape
    if (g.d == 128) {
        launch_short_d<128>(a, g, pl, part, s);
        if (!pl.fused)
            hipLaunchKernelGGL((map_small_reduce_kernel<128>), dim3(rblocks), dim3(256), 0, s, a, part, g.L_tgt, g.H,
                               g.T, pl.KS);
    } else {
        launch_short_d<64>(a, g, pl, part, s);
        if (!pl.fused)
            hipLaunchKernelGGL((map_small_reduce_kernel<64>), dim3(rblocks), dim3(256), 0, s, a, part, g.L_tgt, g.H,
                               g.T, pl.KS);
    }
    return hipGetLastError();
}

}  // namespace kvmap
