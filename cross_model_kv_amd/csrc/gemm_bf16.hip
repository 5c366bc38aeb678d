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
//     reads are bank-conflict free; one barrier per K-step, with W fetched one K-step and
//     X two K-steps ahead of the step being computed;
//   * tile order is XCD-aware: workgroup b runs on XCD b % 8, and each XCD walks
//     "super-tiles" of 8 token blocks x 4 feature tiles of one (t, K|V), so the A rows and
//     the W slab each tile needs are shared through that XCD's L2, and the 8 XCDs work on
//     the same W[t] at the same time (shared through the MALL).

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

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
// by buffer_load_dwordx4 ... lds.  A K-step is two substeps of 32 MFMAs per wave (8 x 4
// blocks of 16 x 16, 32 features deep), one barrier between them.  Each substep is
// written as 8 chunks (the 4 MFMAs of one A block, the fragment reads of the other
// substep's A block and, in 4 of them, of a B block), fenced off from each other, so that
// single loads can sit between chosen chunks and no burst of loads ever stalls a wave's
// MFMA issue:
//   * first substep of K-step kt: MFMAs of its first 32 features; fragment reads of its
//     second 32; the 4 loads of X(kt+2), one every other chunk, into the X buffer that
//     K-step kt-1 used (freed at the last barrier).
//   * wait until this wave's W(kt+1) and X(kt+1) have landed (only X(kt+2) may still be in
//     flight), barrier: K-step kt+1 is visible everywhere and every read of K-step kt is done.
//   * second substep: MFMAs of the second 32 features of K-step kt; fragment reads of the
//     first 32 of K-step kt+1; the 4 loads of W(kt+2), one every other chunk, into the W
//     buffer of K-step kt.
// X -- which misses to HBM on its first touch -- is thus requested about 1.5 K-steps before
// it is needed and W, which the other token blocks of the super-tile keep in L2, one.
// Every K-step issues exactly one W and one X stage in the same order, so every wait count
// is a constant.
//
// 8 waves (two per SIMD): wave w computes features (w & 1) * 128 .. + 127 (whole heads) of
// tokens (w >> 1) * 64 .. + 63.
template <int D>
__global__ __launch_bounds__(512) void map_bf16_kernel(MapArgs a, int L_tgt, int H, int k, int64_t T,
                                                       int nP, int nN) {
    constexpr int NW = 8;                  // waves
    constexpr int TW = 64;                 // tokens per wave
    constexpr int JB = TW / 16;            // 16-token MFMA blocks per wave
    constexpr int LPO = 4;                 // loads per wave per operand per stage (2048 chunks / 64 lanes / NW)
    constexpr int TILE = STAGE_CHUNKS * 16;  // 32 KB: one operand tile of one K-step
    constexpr int NW_BUF = 2, NX_BUF = 3;
    constexpr int MAIN_BYTES = (NW_BUF + NX_BUF) * TILE;
    constexpr int EPI_BYTES = NW * TW * EPI_ROW * 4;
    __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES];
    uint4* lds = (uint4*)smem;  // W buffers 0..1, then X buffers 0..2, 2048 chunks each

    TileId tl;
    if (!decode_tile(blockIdx.x, L_tgt, nP, nN, tl)) return;

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
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);

    // Loads: LDS slot u = i*64*NW + wave*64 + lane of a tile buffer holds row u/8, chunk
    // (u%8) ^ slot_xor(row).  Byte offsets within one K-step, fixed for the whole loop.
    int aoff[LPO], boff[LPO];
#pragma unroll
    for (int i = 0; i < LPO; ++i) {
        const int r = i * 8 * NW + wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        const int n = min(n0 + r, N - 1);
        const int64_t p = min((int64_t)(p0 + r), T - 1);
        // byte offsets below 2^32 (N F < 2^31 and T d < 2^31 are validated): unsigned arithmetic
        aoff[i] = (int)(((uint32_t)n * (uint32_t)F + (uint32_t)c * 8u) * 2u);
        boff[i] = (int)(((uint32_t)p * (uint32_t)D + (uint32_t)c * 8u) * 2u);
    }
    const int nk = F / BK;

    // Issue state of each ring: next buffer, and for W the byte offset of the next K-step,
    // for X the address of the gathered slab (head h of selected layer j, a [T][d] block)
    // and the byte offset of the K-step's 64 features in its rows.  Advanced with adds and
    // selects only, so the loop body has no branches.  Past the last K-step the W offset
    // and j stop at their last values: the extra stages that the branch-free pipeline loads
    // at the end repeat the last one, stay in bounds and are never read.
    //
    // Each stage's issue is planned (buffer, offsets, descriptor: scalar arithmetic only)
    // in a chunk before the ones that issue its loads.
    struct WIssue {
        uint32_t la;
        int soff;
    };
    struct XIssue {
        i32x4_t rsrc;
        uint32_t la;
        int soff;
    };
    const int w_last = (nk - 1) * BK * 2;
    int w_buf = 0, w_soff = 0;
    int x_buf = 0, x_eb = 0, x_h = 0, x_j = 0;
    uint32_t x_lo = (uint32_t)__builtin_amdgcn_readlane(lb_lo, 0);  // slab address, two halves
    uint32_t x_hi = (uint32_t)__builtin_amdgcn_readlane(lb_hi, 0);
    auto plan_w = [&]() {
        const WIssue r = {lds_base + (uint32_t)w_buf * TILE + wave_s * 1024u, w_soff};
        w_buf = (w_buf + 1 == NW_BUF) ? 0 : w_buf + 1;
        w_soff = min(w_soff + BK * 2, w_last);
        return r;
    };
    auto plan_x = [&]() {
        const i32x4_t rs = {(int)x_lo, (int)x_hi, (int)slab_bytes, 0x00020000};
        const XIssue r = {rs, lds_base + (uint32_t)(NW_BUF + x_buf) * TILE + wave_s * 1024u, x_eb};
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
        return r;
    };
    // load i (of LPO) of a stage
    auto issue_w1 = [&](const WIssue& r, int i) { lds_dma16(wr, r.la + i * 1024 * NW, aoff[i], r.soff); };
    auto issue_x1 = [&](const XIssue& r, int i) { lds_dma16(r.rsrc, r.la + i * 1024 * NW, boff[i], r.soff); };
    auto issue_w = [&](const WIssue& r) {
#pragma unroll
        for (int i = 0; i < LPO; ++i) issue_w1(r, i);
    };
    auto issue_x = [&](const XIssue& r) {
#pragma unroll
        for (int i = 0; i < LPO; ++i) issue_x1(r, i);
    };

    // v_mfma_f32_16x16x32_bf16 blocks: IB = 8 blocks of 16 features x JB blocks of 16 tokens.
    // (Per FLOP it moves half the accumulator registers of the 32 x 32 x 16 form.)
    constexpr int IB = 8;
    f32x4_t acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

    const int wn = wave & 1, wp = wave >> 1;
    const int kq = lane >> 4;                       // which 8-feature quarter of a 32-feature substep
    const int fx = slot_xor(lane & 15);             // rows read by this lane: r % 16 = lane % 16
    const int arow = (wn * 128 + (lane & 15)) * 8;  // chunk index of the lane's first A row
    const int brow = (wp * TW + (lane & 15)) * 8;   // ... and of its first B row

    // Fragments of substep ks (0, 1) of a K-step: lane holds row (lane % 16) + 16 i of A block
    // i (B block j), features 32 ks + 8 (lane / 16) .. + 7 of the K-step.
    auto rd_a = [&](int wb, int ks, int i, bf16x8_t* fa) {
        const uint4* la = lds + wb * STAGE_CHUNKS;
        fa[i] = __builtin_bit_cast(bf16x8_t, la[arow + i * 128 + ((ks * 4 + kq) ^ fx)]);
    };
    auto rd_b = [&](int xb, int ks, int j, bf16x8_t* fb) {
        const uint4* lb = lds + (NW_BUF + xb) * STAGE_CHUNKS;
        fb[j] = __builtin_bit_cast(bf16x8_t, lb[brow + j * 128 + ((ks * 4 + kq) ^ fx)]);
    };
    auto mrow = [&](const bf16x8_t* fa, const bf16x8_t* fb, int i) {  // the MFMAs of A block i
#pragma unroll
        for (int j = 0; j < JB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // All waves' loads of a stage are visible once each wave has waited for its own (vmcnt
    // counts the later stages still in flight) and the waves have met at the barrier.  A
    // plain s_barrier: a release fence would add a vmcnt(0) that drains the pipeline.
    auto sync = [&]() {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");  // no LDS read moves above the barrier
    };

    // prologue: W(0) X(0) W(1) X(1); K-step 0 is complete once only W(1) X(1) remain
    issue_w(plan_w());
    issue_x(plan_x());
    issue_w(plan_w());
    issue_x(plan_x());
    XIssue x_next = plan_x();  // X(2), issued during K-step 0
    WIssue w_next;             // W(kt+2), planned during K-step kt
    bf16x8_t fa0[IB], fb0[JB], fa1[IB], fb1[JB];
    wait_vmcnt<2 * LPO>();
    sync();
    int cw = 0, cx = 0;  // ring buffers of the K-step being computed
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        rd_a(cw, 0, i, fa0);
        if (i < JB) rd_b(cx, 0, i, fb0);
    }
    auto kstep = [&]() {  // one K-step
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            rd_a(cw, 1, i, fa1);
            if (i < JB) rd_b(cx, 1, i, fb1);
            mrow(fa0, fb0, i);
            if (i & 1) issue_x1(x_next, i >> 1);  // X(kt+2) -> X buffer of K-step kt-1
            if (i == 2) w_next = plan_w();
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<LPO>();
        sync();
        const int cw1 = (cw + 1 == NW_BUF) ? 0 : cw + 1;
        const int cx1 = (cx + 1 == NX_BUF) ? 0 : cx + 1;
        // (after the last K-step this reads buffers that are never used)
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            if ((i & 1) == 0) issue_w1(w_next, i >> 1);  // W(kt+2) -> W buffer of K-step kt
            rd_a(cw1, 0, i, fa0);
            if (i < JB) rd_b(cx1, 0, i, fb0);
            mrow(fa1, fb1, i);
            if (i == 3) x_next = plan_x();
            __builtin_amdgcn_sched_barrier(0);
        }
        cw = cw1;
        cx = cx1;
    };
    // Two K-steps per trip of the loop (measured 0.4-1.9 % faster than one, same results);
    // an odd count (d = 64 with k H odd) ends with one more.
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
        kstep();
        kstep();
    }
    if (kt < nk) kstep();
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

hipError_t launch_map_bf16(const MapArgs& a, const ApplyGeom& g, int /*cus*/, hipStream_t s) {
    const int N = g.N();
    const int nP = (int)((g.T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int grid = map_bf16_grid(g.L_tgt, g.T, N);
    if (g.d == 128)
        hipLaunchKernelGGL((map_bf16_kernel<128>), dim3(grid), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    else
        hipLaunchKernelGGL((map_bf16_kernel<64>), dim3(grid), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    return hipGetLastError();
}

}  // namespace kvmap
