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

namespace kvmap {

namespace {

constexpr int BM = 256;  // output features per tile
constexpr int BN = 256;  // tokens per tile
constexpr int BK = 64;   // features (reduction) per K-step: one 128-byte line per tile row
constexpr int STAGE_CHUNKS = BM * BK / 8;  // 16-byte chunks per operand per stage (2048)
constexpr int EPI_ROW = 68;                // uint32 words per staged output row (256 B + 16 B pad)

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
    const int tkv = s / spk, sg = s - (s / spk) * spk;
    o.t = tkv >> 1;
    o.kv = tkv & 1;
    o.pb = sg * pg + w / nN;
    o.nb = w - (w / nN) * nN;
    return o.pb < nP;
}

// LDS slot of the 16-byte chunk c (0..7) of tile row r is c ^ slot_xor(r).  Rows are 128
// bytes.  For the rows r..r+15 read by 16 consecutive lanes of a ds_read_b128 (one chunk
// index), (r & 1, c ^ slot_xor(r)) covers all 16 bank groups of a 256-byte (64-bank)
// window, and for 8 consecutive lanes c ^ slot_xor(r) covers the 8 groups of a 128-byte
// window: conflict free under either bank count.
__device__ __forceinline__ int slot_xor(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes) for raw buffer loads (gfx9 dword3 = 0x00020000).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    const i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                       __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)), (int)bytes, 0x00020000};
    return r;
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from rsrc + voff + soff into LDS at
// m0 + 16 * lane.  Written as inline assembly so that the compiler's conservative waits
// for direct-to-LDS loads (it cannot tell the pipeline's stage buffers apart and would
// drain every load before issuing the next stage) stay out of the pipeline; the kernel
// orders these loads itself with explicit vmcnt waits and barriers.  Nothing else in the
// kernel uses m0.
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc, uint32_t lds_addr, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// c ? a : b on uniform values, as one s_cselect.  Written out because the compiler turns a
// select between a v_readlane result and an add into a branch, which would split the loop.
__device__ __forceinline__ uint32_t uniform_select(uint32_t c, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("s_cmp_lg_u32 %1, 0\n\ts_cselect_b32 %0, %2, %3"
        : "=s"(r)
        : "s"(__builtin_amdgcn_readfirstlane(c)), "s"(a), "s"(b)
        : "scc");
    return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N == 0 || N == 4 || N == 8 || N == 12 || N == 16, "vmcnt");  // per-wave loads
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
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
// a 2-deep ring for the W tile and a 3-deep ring for the gathered X tile (160 KB).  Both
// are filled by buffer_load_dwordx4 ... lds: W one K-step ahead, X -- which misses to HBM
// on its first touch -- two K-steps ahead.  A K-step is two substeps of 32 MFMAs per
// wave (8 x 4 blocks of 16 x 16, 32 features deep); the fragments of the next substep are read from LDS
// between the MFMAs of the current one.  Before the second substep a wave waits until its
// loads of K-step kt+1 have landed, meets the other waves at a barrier (K-step kt+1
// visible everywhere, every read of K-step kt done) and issues W(kt+2) and X(kt+3) into
// the buffers K-step kt used.  Every K-step issues exactly one W and one X stage, W
// first, so every wait count is a constant: only X(kt+2) may still be in flight.
//
// NW waves: wave w computes features (w & 1) * 128 .. + 127 (whole heads) of tokens
// (w >> 1) * TW .. + TW - 1, TW = 512 / NW.  With 8 waves (two per SIMD) the load
// instructions one wave stalls on while the memory pipeline drains are covered by the other
// wave's MFMAs.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void map_bf16_kernel(MapArgs a, int L_tgt, int H, int k,
                                                           int64_t T, int nP, int nN) {
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    constexpr int TW = 512 / NW;          // tokens per wave
    constexpr int JB = TW / 16;           // 16-token MFMA blocks per wave
    constexpr int LPO = 32 / NW;          // loads per wave per operand per stage (2048 chunks / 64 lanes / NW)
    constexpr int TILE = STAGE_CHUNKS * 16;            // 32 KB: one operand tile of one K-step
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
        aoff[i] = (n * F + c * 8) * 2;
        boff[i] = ((int)(p * D) + c * 8) * 2;
    }
    const int nk = F / BK;

    // Issue state of each ring: next buffer, and for W the byte offset of the next K-step,
    // for X the address of the gathered slab (head h of selected layer j, a [T][d] block)
    // and the byte offset of the K-step's 64 features in its rows.  Advanced with adds and
    // selects only, so the loop body has no branches.  Past the last K-step the W offset
    // and j stop at their last values: the extra stages that the branch-free pipeline loads
    // at the end repeat the last one, stay in bounds and are never read.
    //
    // Each issue is planned (buffer, offsets, descriptor: scalar arithmetic only) one
    // substep before it is issued, so that after the barrier only the loads themselves stand
    // between the waves and their next MFMAs.
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
        w_buf ^= 1;
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
    auto issue_w = [&](const WIssue& r) {
#pragma unroll
        for (int i = 0; i < LPO; ++i) lds_dma16(wr, r.la + i * 1024 * NW, aoff[i], r.soff);
    };
    auto issue_x = [&](const XIssue& r) {
#pragma unroll
        for (int i = 0; i < LPO; ++i) lds_dma16(r.rsrc, r.la + i * 1024 * NW, boff[i], r.soff);
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

    // Fragments of one 32-feature substep: lane holds rows (lane % 16) + 16 i of its A and B
    // blocks, features 8 * (lane / 16) .. + 7 of the substep.
    auto read_frags = [&](int wb, int xb, int ks, bf16x8_t* fa, bf16x8_t* fb) {
        const uint4* la = lds + wb * STAGE_CHUNKS;
        const uint4* lb = lds + (NW_BUF + xb) * STAGE_CHUNKS;
        const int slot = (ks * 4 + kq) ^ fx;
#pragma unroll
        for (int i = 0; i < IB; ++i) fa[i] = __builtin_bit_cast(bf16x8_t, la[arow + i * 128 + slot]);
#pragma unroll
        for (int j = 0; j < JB; ++j) fb[j] = __builtin_bit_cast(bf16x8_t, lb[brow + j * 128 + slot]);
    };
    auto mfmas = [&](const bf16x8_t* fa, const bf16x8_t* fb) {
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // Interleave: one fragment read after each of the first IB + JB MFMAs of a substep.
    auto interleave = [&]() {
#pragma unroll
        for (int r = 0; r < IB + JB; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, IB * JB - (IB + JB), 0);
    };
    // The same, and then up to two scalar or vector ALU instructions (the planning of the
    // next issue) after each remaining MFMA, so that they never hold the matrix pipe up.
    auto interleave_plan = [&]() {
#pragma unroll
        for (int r = 0; r < IB + JB; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int r = 0; r < IB * JB - (IB + JB); ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
        }
    };
    // All waves' loads of a stage are visible once each wave has waited for its own (vmcnt
    // counts the later stages still in flight) and the waves have met at the barrier.  A
    // plain s_barrier: a release fence would add a vmcnt(0) that drains the pipeline.
    auto sync = [&]() {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");  // no LDS read moves above the barrier
    };

    // prologue: W(0) X(0) W(1) X(1) X(2); K-step 0 complete once only W(1) X(1) X(2) remain
    issue_w(plan_w());
    issue_x(plan_x());
    issue_w(plan_w());
    issue_x(plan_x());
    issue_x(plan_x());
    WIssue w_next = plan_w();  // W(2) and X(3): the first issues inside the loop
    XIssue x_next = plan_x();
    bf16x8_t fa0[IB], fb0[JB], fa1[IB], fb1[JB];
    wait_vmcnt<3 * LPO>();
    sync();
    int cw = 0, cx = 0;  // ring buffers of the K-step being computed
    read_frags(cw, cx, 0, fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
        read_frags(cw, cx, 1, fa1, fb1);
        mfmas(fa0, fb0);
        interleave();
        // All reads of K-step kt are issued; once they have returned and K-step kt+1 has
        // landed (only X(kt+2) may be outstanding), the barrier frees K-step kt's buffers.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<LPO>();
        sync();
        issue_w(w_next);  // W(kt+2) -> W buffer of K-step kt
        issue_x(x_next);  // X(kt+3) -> X buffer of K-step kt
        cw ^= 1;
        cx = (cx + 1 == NX_BUF) ? 0 : cx + 1;
        // (after the last K-step this reads buffers that are never used)
        read_frags(cw, cx, 0, fa0, fb0);
        mfmas(fa1, fb1);
        w_next = plan_w();
        x_next = plan_x();
        interleave();
    }
    wait_vmcnt<0>();  // the extra tail stages must land before LDS is reused below
    __syncthreads();  // every wave is done reading the pipeline buffers

    // ---- epilogue: + bias, target RoPE on keys, bf16 -> LDS (per-wave [TW tokens][128
    // features], padded rows), then full 256-byte rows to the target cache [t][h][p][e] ----
    // Lane holds D[n][p] for p = col (lane & 15) and n = 4 * (lane / 16) + r of each 16 x 16
    // block: 4 consecutive features -> one 8-byte LDS store.
    constexpr int HALF = D / 2;
    constexpr int PB = HALF / 16;  // block distance between the two members of a RoPE pair
    const uint16_t* __restrict__ bias = (const uint16_t*)(tl.kv ? a.bv : a.bk) + (size_t)tl.t * N;
    uint16_t* __restrict__ out = (uint16_t*)(tl.kv ? a.outv : a.outk);
    const int nw = n0 + wn * 128;
    const int pw = p0 + wp * TW;
    const bool rope = (tl.kv == 0);
    uint32_t* stg = (uint32_t*)smem + wave * (TW * EPI_ROW);
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        if ((i / PB) & 1) continue;  // i is the low member; i + PB the high one
        const int nl = i * 16 + kq * 4;  // feature offset in the wave (low member)
        const int nlo = min(nw + nl, N - 4), nhi = nlo + HALF;
        const int elo = nlo % D;
        const uint2 blo = *(const uint2*)(bias + nlo);
        const uint2 bhi = *(const uint2*)(bias + nhi);
        const float bl[4] = {bf16lo(blo.x), bf16hi(blo.x), bf16lo(blo.y), bf16hi(blo.y)};
        const float bh[4] = {bf16lo(bhi.x), bf16hi(bhi.x), bf16lo(bhi.y), bf16hi(bhi.y)};
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int pl = j * 16 + (lane & 15);
            const int64_t p = min((int64_t)(pw + pl), T - 1);
            float ylo[4], yhi[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ylo[r] = acc[i][j][r] + bl[r];
                yhi[r] = acc[i + PB][j][r] + bh[r];
            }
            if (rope) {
                const float4* cs4 = (const float4*)(a.tab_tgt + p * HALF + elo);
                const float4 c01 = cs4[0], c23 = cs4[1];
                const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
                const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float l = ylo[r], hh = yhi[r];
                    ylo[r] = fmaf(-hh, ss[r], l * cc[r]);
                    yhi[r] = fmaf(l, ss[r], hh * cc[r]);
                }
            }
            uint32_t* row = stg + pl * EPI_ROW;
            *(uint2*)(row + nl / 2) = make_uint2(pack_bf16(ylo[0], ylo[1]), pack_bf16(ylo[2], ylo[3]));
            *(uint2*)(row + (nl + HALF) / 2) = make_uint2(pack_bf16(yhi[0], yhi[1]), pack_bf16(yhi[2], yhi[3]));
        }
    }
    __syncthreads();
    // 16 lanes per staged row, 16 bytes each: 4 full rows per store instruction.
#pragma unroll 4
    for (int it = 0; it < TW / 4; ++it) {
        const int pl = it * 4 + (lane >> 4);
        const int c = lane & 15;                    // 16-byte chunk = features c*8 .. c*8+7
        const int64_t p = pw + pl;
        const int n = nw + c * 8;
        if (p >= T || n >= N) continue;
        const int h = n / D, e = n - h * D;
        const uint4 v = *(const uint4*)(stg + pl * EPI_ROW + c * 4);
        *(uint4*)(out + (((size_t)tl.t * H + h) * T + p) * D + e) = v;
    }
}

#ifndef KVMAP_MAP_WAVES
#define KVMAP_MAP_WAVES 8
#endif

hipError_t launch_map_bf16(const MapArgs& a, const ApplyGeom& g, hipStream_t s) {
    const int N = g.N();
    const int nP = (int)((g.T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int grid = map_bf16_grid(g.L_tgt, g.T, N);
    constexpr int NW = KVMAP_MAP_WAVES;
    if (g.d == 128)
        hipLaunchKernelGGL((map_bf16_kernel<128, NW>), dim3(grid), dim3(64 * NW), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    else
        hipLaunchKernelGGL((map_bf16_kernel<64, NW>), dim3(grid), dim3(64 * NW), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    return hipGetLastError();
}

}  // namespace kvmap
