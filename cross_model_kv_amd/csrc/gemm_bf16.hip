// The map GEMM for bf16 caches: for every target layer t and both K and V,
//   Y[p, n] = sum_f X[p, f] * W[t][n][f] + b[t][n],   X[p, (j*H + h)*d + e] = src[sel[t][j]][h][p][e]
// with fp32 accumulation on the gfx950 matrix cores, the bias add and (for keys) the
// target-model RoPE fused into the epilogue, and bf16 output written straight into the
// target cache layout [t][h][p][e].  The gather is free: one K-step of 64 features always
// lies inside one (selected layer, source head) slab, which is a contiguous [T][d] block,
// so the tile's base pointer changes per K-step and its rows are plain strided loads.
//
// Mapping of the work (VeloxQuant-MLX "Cross-Model KV Transfer", "The mapping": one ridge map
// per target head, for K and for V; KVBridge README "What ships": cross-head features):
//   * output tile 256 features x 256 tokens per workgroup of 8 waves (2 x 4), each wave
//     128 features x 64 tokens; a wave's 128 features are whole heads, so both members
//     (e, e + d/2) of every RoPE pair sit in the same lane;
//   * v_mfma_f32_16x16x32_bf16 (gfx950): A = W rows (features), B = X rows (tokens),
//     both K-contiguous in memory and in LDS;
//   * K-steps of 64 features, so every tile row is one whole 128-byte line; the stages are
//     filled straight from HBM by buffer_load ... lds into two LDS rings, 2 stages for W and
//     3 for X (5 x 32 KB), with 16-byte chunks XOR-swizzled by row so the MFMA fragment
//     reads are bank-conflict free;
//   * the two groups of 4 waves (one wave of each per SIMD) take turns: one issues a K-step's
//     MFMAs back to back while the other reads its next fragments and issues the loads, so no
//     memory instruction ever sits between a wave's MFMAs;
//   * tile order is XCD-aware: workgroup b runs on XCD b % 8, and each XCD walks
//     "super-tiles" of 8 token blocks x 4 feature tiles of one (t, K|V), so the A rows and
//     the W slab each tile needs are shared through that XCD's L2, and the 8 XCDs work on
//     the same W[t] at the same time (shared through the MALL).

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

#include <algorithm>

namespace kvmap {

namespace {

constexpr int BM = 256;  // output features per tile
constexpr int BN = 256;  // tokens per tile
constexpr int BK = 64;   // features (reduction) per K-step: one 128-byte line per tile row
constexpr int STAGE_CHUNKS = BM * BK / 8;  // 16-byte chunks per operand per stage (2048)
constexpr int EPI_ROW = 68;                // uint32 words per staged output row (256 B + 16 B pad)

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

struct TileId {
    int t, kv, pb, nb;
};

// blockIdx -> tile, grouping tiles into per-XCD super-tiles (see file comment).
__device__ __forceinline__ bool decode_tile(int bid, int L_tgt, int nP, int nN, TileId& o) {
    const int pg = nN >= 32 ? 1 : 32 / nN;  // token blocks per super-tile
    const int spk = (nP + pg - 1) / pg;     // super-tiles per (t, kv)
    const int S = L_tgt * 2 * spk;
    const int tps = pg * nN;                // tiles per super-tile
    const int xcd = bid & 7, local = bid >> 3;
    const int s = (local / tps) * 8 + xcd;
    const int w = local - (local / tps) * tps;
    if (s >= S) return false;
    // (t, K|V) pairs.  With fewer than 8 super-tiles per pair (caches of up to 14,336 tokens)
    // the 8 XCDs work on different pairs at once: then every target layer's keys come first,
    // then every target layer's values, so that the pairs in flight read one contiguous span of
    // one map tensor (alternating the K and V maps, two allocations read at the same offsets in
    // lockstep, streams W up to 25 % slower).  With 8 or more, all XCDs share one pair at a
    // time, and t-major order (K then V of each target layer) measured 2 % faster.
    const int tkv = s / spk, sg = s - (s / spk) * spk;
    if (spk < 8) {
        o.kv = tkv / L_tgt;
        o.t = tkv - o.kv * L_tgt;
    } else {
        o.t = tkv >> 1;
        o.kv = tkv & 1;
    }
    o.pb = sg * pg + w / nN;
    o.nb = w - (w / nN) * nN;
    return o.pb < nP;
}

}  // namespace

int map_bf16_grid(int L_tgt, int64_t T, int N) {
    const int nP = (int)((T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int pg = nN >= 32 ? 1 : 32 / nN;
    const int spk = (nP + pg - 1) / pg;
    const int S = L_tgt * 2 * spk;
    return ((S + 7) / 8) * pg * nN * 8;
}

// Software pipeline over K-steps of 64 features (one 128-byte line per tile row, so every
// 8 lanes of a load cover a whole cache line).  LDS holds two rings of 32 KB tile buffers:
// a 2-deep ring for the W tile and a 3-deep ring for the gathered X tile (160 KB), filled
// by buffer_load_dwordx4 ... lds; the schedule is the ping-pong of the two wave groups
// described in the kernel.  X -- which misses to HBM on its first touch -- is requested
// about 1.5 K-steps before it is needed and W, which the other token blocks of the
// super-tile keep in L2, one.
//
// 8 waves (two per SIMD): wave w computes features (w & 1) * 128 .. + 127 (whole heads) of
// tokens (w >> 1) * 64 .. + 63.
template <int D>
__device__ __forceinline__ void map_tile(const MapArgs& a, int L_tgt, int H, int k, int64_t T,
                                         const TileId& tl, char* smem, uint32_t lds_base) {
    constexpr int NW = 8;                  // waves
    constexpr int TW = 64;                 // tokens per wave
    constexpr int JB = TW / 16;            // 16-token MFMA blocks per wave
    constexpr int TILE = STAGE_CHUNKS * 16;  // 32 KB: one operand tile of one K-step
    constexpr int NW_BUF = 2, NX_BUF = 3;
    constexpr int MAIN_BYTES = (NW_BUF + NX_BUF) * TILE;
    constexpr int EPI_BYTES = NW * TW * EPI_ROW * 4;
    uint4* lds = (uint4*)smem;  // W buffers 0..1, then X buffers 0..2, 2048 chunks each
    const int N = H * D, F = k * N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = tl.nb * BM, p0 = tl.pb * BN;
    const uint16_t* __restrict__ X = (const uint16_t*)(tl.kv ? a.xv : a.xk);
    const uint16_t* __restrict__ W = (const uint16_t*)(tl.kv ? a.Wv : a.Wk) + (size_t)tl.t * N * F;
    // Lane j keeps the address of head 0 of selected source layer j of this target layer
    // (k <= 64); the loop reads it back with v_readlane, so it issues no memory load besides
    // the pipeline's own.
    const size_t slab = (size_t)T * D;
    const uint32_t slab_bytes = (uint32_t)(slab * 2);
    const uint64_t lbase = (uint64_t)(uintptr_t)(X + (size_t)(lane < k ? a.sel[tl.t * k + lane] : 0) * H * slab);
    const int lb_lo = (int)(uint32_t)lbase, lb_hi = (int)(uint32_t)(lbase >> 32);
    const i32x4_t wr = make_rsrc(W, (uint32_t)((size_t)N * F * 2));

    // The 8 waves form two groups of 4, one wave of each group per SIMD (waves 0-3 and 4-7).
    // The groups take turns: while one group issues its 64 MFMAs of a K-step back to back, the
    // other reads its fragments of the next K-step from LDS and issues global loads; one
    // barrier ends every such phase.  Group 0 runs one phase ahead of group 1:
    //   phase 2kt     group 0: loads W(kt+1), reads K-step kt    group 1: MFMAs of K-step kt-1
    //   phase 2kt+1   group 0: MFMAs of K-step kt                 group 1: loads X(kt+2), reads kt
    // so each SIMD's matrix pipe is fed by one wave's run of independent MFMAs at a time, and
    // no load or LDS read is ever issued between them.  Group 0 loads the W stages (8 loads per
    // wave per stage), group 1 the X stages.  Rings: W 2 deep, X 3 deep (160 KB).  W(kt+1)
    // goes into the buffer that K-step kt-1 used, free once group 1 read it in phase 2kt-1;
    // X(kt+2) into K-step kt-1's, also free.  Stage kt+1 is complete at the barrier ending
    // phase 2kt+1: group 0 waits for its W(kt+1) at the end of its MFMA phase, group 1 for its
    // X(kt+1) at the end of its read phase (only X(kt+2) may still be in flight).  Group 1
    // passes one extra barrier first (phase 0, when only group 0 works), group 0 one last.
    constexpr int LPG = 8;  // loads per wave per stage of its group's operand (2048 chunks / 256 lanes)
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2), wig = wave & 3;  // uniform per wave
    const uint32_t wig_s = __builtin_amdgcn_readfirstlane(wig);
    // Loads: LDS slot u = i*256 + wig*64 + lane of a tile buffer holds row u/8, chunk
    // (u%8) ^ slot_xor(row).  Byte offsets within one K-step, fixed for the whole loop.
    int loff[LPG];
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
        const int r = i * 32 + wig * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        const int n = min(n0 + r, N - 1);
        const int64_t p = min((int64_t)(p0 + r), T - 1);
        // byte offsets below 2^32 (N F < 2^31 and T d < 2^31 are validated): unsigned arithmetic
        loff[i] = grp == 0 ? (int)(((uint32_t)n * (uint32_t)F + (uint32_t)c * 8u) * 2u)
                           : (int)(((uint32_t)p * (uint32_t)D + (uint32_t)c * 8u) * 2u);
    }
    const int nk = F / BK;

    constexpr int IB = 8;
    f32x4_t acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

    const int wn = wave & 1, wp = wave >> 1;
    const int kq = lane >> 4;
    const int fx = slot_xor(lane & 15);
    const int arow = (wn * 128 + (lane & 15)) * 8;
    const int brow = (wp * TW + (lane & 15)) * 8;
    bf16x8_t fa[2][IB], fb[2][JB];
    auto read_stage = [&](int wb, int xb) {
        const uint4* la = lds + wb * STAGE_CHUNKS;
        const uint4* lb = lds + (NW_BUF + xb) * STAGE_CHUNKS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < IB; ++i) fa[ks][i] = __builtin_bit_cast(bf16x8_t, la[arow + i * 128 + ((ks * 4 + kq) ^ fx)]);
#pragma unroll
            for (int j = 0; j < JB; ++j) fb[ks][j] = __builtin_bit_cast(bf16x8_t, lb[brow + j * 128 + ((ks * 4 + kq) ^ fx)]);
        }
    };
    auto mfma_stage = [&]() {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };
    auto sync = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");  // no LDS read moves above the barrier
        __builtin_amdgcn_sched_barrier(0);
    };

    if (grp == 0) {
        // W stages: buffer kt % 2, byte offset kt * 128 of every W row (the last K-step's
        // offset repeated past the end: those stages stay in bounds and are never read)
        const int w_last = (nk - 1) * BK * 2;
        auto issue_w = [&](int kt) {
            const uint32_t la = lds_base + (uint32_t)(kt & 1) * TILE + wig_s * 1024u;
            const int soff = min(kt * BK * 2, w_last);
#pragma unroll
            for (int i = 0; i < LPG; ++i) lds_dma16(wr, la + i * 4096, loff[i], soff);
        };
        issue_w(0);
        wait_vmcnt<0>();
        sync();  // stage 0 complete
        for (int kt = 0; kt < nk; ++kt) {
            issue_w(kt + 1);
            read_stage(kt & 1, kt % 3);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            sync();
            mfma_stage();
            wait_vmcnt<0>();  // W(kt+1) landed
            sync();
        }
        sync();  // group 1's last MFMA phase
    } else {
        // X stages: buffer kt % 3, the gathered slab (head h of selected layer j: a [T][d]
        // block) and the byte offset of the K-step's 64 features in its rows, advanced with
        // adds and selects only; past the last K-step j stays at its last value.
        int x_buf = 0, x_eb = 0, x_h = 0, x_j = 0;
        uint32_t x_lo = (uint32_t)__builtin_amdgcn_readlane(lb_lo, 0);
        uint32_t x_hi = (uint32_t)__builtin_amdgcn_readlane(lb_hi, 0);
        auto issue_x = [&]() {
            const i32x4_t rs = {(int)x_lo, (int)x_hi, (int)slab_bytes, 0x00020000};
            const uint32_t la = lds_base + (uint32_t)(NW_BUF + x_buf) * TILE + wig_s * 1024u;
#pragma unroll
            for (int i = 0; i < LPG; ++i) lds_dma16(rs, la + i * 4096, loff[i], x_eb);
            x_buf = (x_buf + 1 == NX_BUF) ? 0 : x_buf + 1;
            x_eb += BK * 2;
            const int we = (x_eb == D * 2);  // next head
            x_eb = we ? 0 : x_eb;
            x_h += we;
            const int wh = (x_h == H);  // next selected layer
            x_h = wh ? 0 : x_h;
            x_j = min(x_j + wh, k - 1);
            const uint32_t a_lo = x_lo + (we ? slab_bytes : 0u);
            const uint32_t a_hi = x_hi + (a_lo < x_lo ? 1u : 0u);
            x_lo = uniform_select(wh, (uint32_t)__builtin_amdgcn_readlane(lb_lo, x_j), a_lo);
            x_hi = uniform_select(wh, (uint32_t)__builtin_amdgcn_readlane(lb_hi, x_j), a_hi);
        };
        issue_x();  // X(0)
        issue_x();  // X(1)
        wait_vmcnt<LPG>();
        sync();  // stage 0 complete
        sync();  // phase 0: group 0 reads stage 0
        for (int kt = 0; kt < nk; ++kt) {
            issue_x();  // X(kt+2)
            read_stage(kt & 1, kt % 3);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            wait_vmcnt<LPG>();  // X(kt+1) landed
            sync();
            mfma_stage();
            sync();
        }
    }
    wait_vmcnt<0>();  // the extra tail stages must land before LDS is reused below
    __syncthreads();  // every wave is done reading the pipeline buffers

    // ---- epilogue: + bias, target RoPE on keys, bf16 -> LDS (per-wave [TW tokens][128
    // features], padded rows), then full 256-byte rows to the target cache [t][h][p][e] ----
    // Lane holds D[n][p] for p = col (lane & 15) and n = 4 * (lane / 16) + r of each 16 x 16
    // block: 4 consecutive features -> one 8-byte LDS store.  Each wave stages and stores only
    // its own rows, so no barrier is needed between the two phases.
    constexpr int HALF = D / 2;
    constexpr int PB = HALF / 16;  // block distance between the two members of a RoPE pair
    constexpr int NLO = IB / 2;    // blocks holding low members: i = lo_block(li)
    constexpr int JC = 2;          // token blocks whose table entries are loaded together
    const uint16_t* __restrict__ bias = (const uint16_t*)(tl.kv ? a.bv : a.bk) + (size_t)tl.t * N;
    uint16_t* __restrict__ out = (uint16_t*)(tl.kv ? a.outv : a.outk);
    const int nw = n0 + wn * 128;
    const int pw = p0 + wp * TW;
    uint32_t* stg = (uint32_t*)smem + wave * (TW * EPI_ROW);
    auto lo_block = [](int li) { return (li / PB) * 2 * PB + li % PB; };
    // A block's head lies inside the target cache or wholly past its last head (partial last
    // feature tile); the latter is neither read from the bias nor stored.
    auto head_ok = [&](int i) { return nw + (i * 16 / D) * D < N; };

    auto finish = [&](auto rope_tag) {
        constexpr bool ROPE = decltype(rope_tag)::value;
        uint2 blo[NLO], bhi[NLO];
#pragma unroll
        for (int li = 0; li < NLO; ++li) {
            const int i = lo_block(li);
            const int n = nw + i * 16 + kq * 4;
            blo[li] = head_ok(i) ? *(const uint2*)(bias + n) : make_uint2(0, 0);
            bhi[li] = head_ok(i) ? *(const uint2*)(bias + n + HALF) : make_uint2(0, 0);
        }
#pragma unroll
        for (int jc = 0; jc < JB; jc += JC) {
            float4 cs[JC][NLO][2];  // (cos, sin) of the lane's 4 pairs per block
            if constexpr (ROPE) {
#pragma unroll
                for (int jj = 0; jj < JC; ++jj) {
                    const int64_t p = min((int64_t)(pw + (jc + jj) * 16 + (lane & 15)), T - 1);
#pragma unroll
                    for (int li = 0; li < NLO; ++li) {
                        const int elo = (lo_block(li) * 16 + kq * 4) % D;
                        const float4* c4 = (const float4*)(a.tab_tgt + p * HALF + elo);
                        cs[jj][li][0] = c4[0];
                        cs[jj][li][1] = c4[1];
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < JC; ++jj) {
                const int j = jc + jj;
                const int pl = j * 16 + (lane & 15);
                uint32_t* row = stg + pl * EPI_ROW;
#pragma unroll
                for (int li = 0; li < NLO; ++li) {
                    const int i = lo_block(li);
                    const int nl = i * 16 + kq * 4;
                    float ylo[4], yhi[4];
                    const float bl[4] = {bf16lo(blo[li].x), bf16hi(blo[li].x), bf16lo(blo[li].y), bf16hi(blo[li].y)};
                    const float bh[4] = {bf16lo(bhi[li].x), bf16hi(bhi[li].x), bf16lo(bhi[li].y), bf16hi(bhi[li].y)};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ylo[r] = acc[i][j][r] + bl[r];
                        yhi[r] = acc[i + PB][j][r] + bh[r];
                    }
                    if constexpr (ROPE) {
                        const float4 c01 = cs[jj][li][0], c23 = cs[jj][li][1];
                        const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
                        const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float l = ylo[r], hh = yhi[r];
                            ylo[r] = fmaf(-hh, ss[r], l * cc[r]);
                            yhi[r] = fmaf(l, ss[r], hh * cc[r]);
                        }
                    }
                    *(uint2*)(row + nl / 2) = make_uint2(pack_bf16(ylo[0], ylo[1]), pack_bf16(ylo[2], ylo[3]));
                    *(uint2*)(row + (nl + HALF) / 2) =
                        make_uint2(pack_bf16(yhi[0], yhi[1]), pack_bf16(yhi[2], yhi[3]));
                }
            }
        }
    };
    if (tl.kv == 0)
        finish(BoolTag<true>{});
    else
        finish(BoolTag<false>{});

    // 16 lanes per staged row, 16 bytes each: 4 full rows per store instruction.
    const int c = lane & 15;  // 16-byte chunk = features c*8 .. c*8+7 of the wave's 128
    if (pw + TW <= T && nw + 128 <= N) {
        const int h = (nw + c * 8) / D, e = (nw + c * 8) % D;
        uint16_t* dst = out + (((size_t)tl.t * H + h) * T + pw + (lane >> 4)) * D + e;
        uint4 v[TW / 4];
#pragma unroll
        for (int it = 0; it < TW / 4; ++it) v[it] = *(const uint4*)(stg + (it * 4 + (lane >> 4)) * EPI_ROW + c * 4);
#pragma unroll
        for (int it = 0; it < TW / 4; ++it) *(uint4*)(dst + (size_t)it * 4 * D) = v[it];
    } else {
#pragma unroll 4
        for (int it = 0; it < TW / 4; ++it) {
            const int pl = it * 4 + (lane >> 4);
            const int64_t p = pw + pl;
            const int n = nw + c * 8;
            if (p >= T || n >= N) continue;
            const int h = n / D, e = n - h * D;
            const uint4 v = *(const uint4*)(stg + pl * EPI_ROW + c * 4);
            *(uint4*)(out + (((size_t)tl.t * H + h) * T + p) * D + e) = v;
        }
    }
}

// Persistent over tiles: workgroup b takes tiles b, b + G, b + 2G, ... of the XCD-aware order
// (G = gridDim.x, a multiple of 8, so a workgroup's tiles are all on its own XCD and in the same
// position of successive super-tiles).  The 32 workgroups of an XCD thus start every super-tile
// together, so the 4 feature tiles that share a token block's X rows stay in step through
// that XCD's L2, instead of starting whenever a compute unit frees up.
template <int D>
__global__ __launch_bounds__(512) void map_bf16_kernel(MapArgs a, int L_tgt, int H, int k, int64_t T,
                                                       int nP, int nN, int total) {
    constexpr int NW = 8;                  // waves
    constexpr int TW = 64;                 // tokens per wave
    constexpr int JB = TW / 16;            // 16-token MFMA blocks per wave
    constexpr int TILE = STAGE_CHUNKS * 16;  // 32 KB: one operand tile of one K-step
    constexpr int NW_BUF = 2, NX_BUF = 3;
    constexpr int MAIN_BYTES = (NW_BUF + NX_BUF) * TILE;
    constexpr int EPI_BYTES = NW * TW * EPI_ROW * 4;
    __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES];
    for (int bid = blockIdx.x; bid < total; bid += gridDim.x) {
        TileId tl;
        if (!decode_tile(bid, L_tgt, nP, nN, tl)) continue;
        map_tile<D>(a, L_tgt, H, k, T, tl, smem, (uint32_t)(uintptr_t)(lds_ptr_t)smem);
        __syncthreads();  // the next tile's loads overwrite LDS that this tile's epilogue read
    }
}

hipError_t launch_map_bf16(const MapArgs& a, const ApplyGeom& g, int cus, hipStream_t s) {
    const int N = g.N();
    const int nP = (int)((g.T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int total = map_bf16_grid(g.L_tgt, g.T, N);  // a multiple of 8
    // Persistent (one workgroup per compute unit) only when every super-tile is whole: 32 tiles,
    // all valid.  Otherwise (caches of a few token blocks, odd head counts) the super-tiles have
    // empty or missing slots, and a workgroup per tile keeps the work spread over the chip.
    const int pg = nN >= 32 ? 1 : 32 / nN;
    const bool whole = pg * nN == 32 && nP % pg == 0;
    const int grid = whole ? std::max(8, std::min(total, (cus / 8) * 8)) : total;
    if (g.d == 128)
        hipLaunchKernelGGL((map_bf16_kernel<128>), dim3(grid), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN, total);
    else
        hipLaunchKernelGGL((map_bf16_kernel<64>), dim3(grid), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN, total);
    return hipGetLastError();
}

}  // namespace kvmap
