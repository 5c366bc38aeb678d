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
//   * output tile 256 features x 256 tokens, 4 waves of 128 x 128; a wave's 128 features
//     are whole heads, so both members (e, e + d/2) of every RoPE pair sit in the same lane;
//   * v_mfma_f32_32x32x16_bf16 (gfx950): A = W rows (features), B = X rows (tokens),
//     both K-contiguous in memory and in LDS;
//   * LDS double buffer (2 x 64 KB) filled straight from HBM by buffer_load ... lds, 16-byte
//     chunks XOR-swizzled by row so the MFMA fragment reads are bank-conflict free; one
//     barrier per K-step;
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

// Two-stage software pipeline over K-steps of 64 features (one 128-byte line per tile row,
// so every 8 lanes of a load cover a whole cache line).  Stage kt lives in LDS buffer
// kt % 2 and is filled by buffer_load_dwordx4 ... lds issued one K-step ahead (8 loads per
// wave per stage: 4 for the W tile, 4 for the X tile).  A K-step is four substeps of 8
// MFMAs per wave; the fragments of the next substep are read from LDS between the MFMAs
// of the current one.  Before the last substep a wave waits until its loads of stage kt+1
// have landed, meets the other waves at a barrier (all loads of stage kt+1 visible, all
// reads of stage kt done) and issues stage kt+2 into the buffer stage kt used.  Every
// K-step issues exactly one stage, so every wait count is a constant.
//
// 8 waves, two per SIMD: wave w computes features (w & 1) * 128 .. + 127 (whole heads) of
// tokens (w >> 1) * 64 .. + 63.  With two waves per SIMD, the load instructions one wave
// stalls on while the memory pipeline drains are covered by the other wave's MFMAs.
template <int D, int NS>
__global__ __launch_bounds__(512) void map_bf16_kernel(MapArgs a, int L_tgt, int H, int k,
                                                       int64_t T, int nP, int nN) {
    static_assert(NS == 2, "two LDS stages of 64 KB");
    constexpr int LOADS = 8;  // per wave per stage
    constexpr int MAIN_BYTES = NS * 2 * STAGE_CHUNKS * 16;
    constexpr int EPI_BYTES = 8 * 64 * EPI_ROW * 4;
    __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES];
    uint4* lds = (uint4*)smem;  // [stage][A=W | B=X][2048 chunks]

    TileId tl;
    if (!decode_tile(blockIdx.x, L_tgt, nP, nN, tl)) return;

    const int N = H * D, F = k * N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = tl.nb * BM, p0 = tl.pb * BN;
    const uint16_t* __restrict__ X = (const uint16_t*)(tl.kv ? a.xv : a.xk);
    const uint16_t* __restrict__ W = (const uint16_t*)(tl.kv ? a.Wv : a.Wk) + (size_t)tl.t * N * F;
    // Lane j keeps selected source layer j of this target layer (k <= 64); a K-step reads it
    // back with v_readlane, so the loop issues no memory load besides the pipeline's own.
    const int selv = lane < k ? a.sel[tl.t * k + lane] : 0;
    const size_t slab = (size_t)T * D;
    const uint32_t slab_bytes = (uint32_t)(slab * 2);
    const i32x4_t wr = make_rsrc(W, (uint32_t)((size_t)N * F * 2));
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);

    // Loads: LDS slot u = i*512 + wave*64 + lane of a stage holds row u/8, chunk
    // (u%8) ^ slot_xor(row).  Byte offsets within one K-step, fixed for the whole loop.
    int aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = i * 64 + wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        const int n = min(n0 + r, N - 1);
        const int64_t p = min((int64_t)(p0 + r), T - 1);
        aoff[i] = (n * F + c * 8) * 2;
        boff[i] = ((int)(p * D) + c * 8) * 2;
    }
    const int nk = F / BK;

    // Issue state: LDS buffer, W byte offset and gathered-slab position (element e within
    // head h of selected layer j) of the next K-step to load.  Advanced with selects only,
    // so the loop body has no branches.  Past the last K-step the W loads fall outside the
    // buffer range (the hardware returns zeros) and j is clamped, so the extra stages the
    // branch-free pipeline loads at the end are harmless and never read.
    int i_stage = 0, i_soff = 0, i_e = 0, i_h = 0, i_j = 0;
    auto issue_next = [&]() {
        const int l1 = __builtin_amdgcn_readlane(selv, min(i_j, k - 1));
        const i32x4_t xr = make_rsrc(X + ((size_t)l1 * H + i_h) * slab + i_e, slab_bytes);
        const uint32_t la = lds_base + (uint32_t)i_stage * (2 * STAGE_CHUNKS * 16) + wave_s * 1024u;
        const uint32_t lb = la + STAGE_CHUNKS * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lds_dma16(wr, la + i * 8192, aoff[i], i_soff);
            lds_dma16(xr, lb + i * 8192, boff[i], 0);
        }
        i_stage ^= 1;
        i_soff += BK * 2;
        i_e += BK;
        const int we = (i_e == D);
        i_e = we ? 0 : i_e;
        i_h += we;
        const int wh = (i_h == H);
        i_h = wh ? 0 : i_h;
        i_j += wh;
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int wn = wave & 1, wp = wave >> 1;
    const int khalf = lane >> 5;
    const int fx = slot_xor(lane & 31);             // rows read by this lane: r % 32 = lane % 32
    const int arow = (wn * 128 + (lane & 31)) * 8;  // chunk index of the lane's first A row
    const int brow = (wp * 64 + (lane & 31)) * 8;   // ... and of its first B row

    // Fragments of one 16-feature substep: lane holds rows (lane % 32) + 32 i of its A and B
    // blocks, features 8 * (lane / 32) .. + 7 of the substep.
    auto read_frags = [&](int stage, int ks, bf16x8_t* fa, bf16x8_t* fb) {
        const uint4* la = lds + (stage * 2) * STAGE_CHUNKS;
        const uint4* lb = la + STAGE_CHUNKS;
        const int slot = (ks * 2 + khalf) ^ fx;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = __builtin_bit_cast(bf16x8_t, la[arow + i * 256 + slot]);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = __builtin_bit_cast(bf16x8_t, lb[brow + j * 256 + slot]);
    };
    auto mfmas = [&](const bf16x8_t* fa, const bf16x8_t* fb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // Interleave: one fragment read after each of the first 6 MFMAs of a substep.
    auto interleave = [&]() {
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };
    // All waves' loads of a stage are visible once each wave has waited for its own (vmcnt
    // counts the later stages still in flight) and the waves have met at the barrier.  A
    // plain s_barrier: a release fence would add a vmcnt(0) that drains the pipeline.
    auto sync = [&]() {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");  // no LDS read moves above the barrier
    };

    issue_next();  // stage 0 -> buffer 0
    issue_next();  // stage 1 -> buffer 1
    bf16x8_t fa0[4], fb0[2], fa1[4], fb1[2];
    wait_vmcnt<LOADS>();
    sync();
    read_frags(0, 0, fa0, fb0);
    int cs = 0;  // LDS buffer of the K-step being computed
    for (int kt = 0; kt < nk; ++kt) {
        read_frags(cs, 1, fa1, fb1);
        mfmas(fa0, fb0);
        interleave();
        read_frags(cs, 2, fa0, fb0);
        mfmas(fa1, fb1);
        interleave();
        read_frags(cs, 3, fa1, fb1);
        mfmas(fa0, fb0);
        interleave();
        // All reads of stage kt are issued; once they have returned, and stage kt+1 has
        // landed, the barrier frees buffer cs for stage kt+2.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<0>();
        sync();
        issue_next();
        cs ^= 1;
        // (after the last K-step this reads a buffer that is never used)
        read_frags(cs, 0, fa0, fb0);
        mfmas(fa1, fb1);
        interleave();
    }
    wait_vmcnt<0>();  // the extra tail stages must land before LDS is reused below
    __syncthreads();  // every wave is done reading the pipeline buffers

    // ---- epilogue: + bias, target RoPE on keys, bf16 -> LDS (per-wave [64 tokens][128
    // features], padded rows), then full 256-byte rows to the target cache [t][h][p][e] ----
    // Lane holds D[n][p] for p = col (lane & 31) and n = 8*(r/4) + 4*(lane/32) + r%4 of each
    // 32x32 block: 4 consecutive features per register group.
    constexpr int HALF = D / 2;
    constexpr int PB = HALF / 32;  // block distance between the two members of a pair
    const uint16_t* __restrict__ bias = (const uint16_t*)(tl.kv ? a.bv : a.bk) + (size_t)tl.t * N;
    uint16_t* __restrict__ out = (uint16_t*)(tl.kv ? a.outv : a.outk);
    const int nw = n0 + wn * 128;
    const int pw = p0 + wp * 64;
    const bool rope = (tl.kv == 0);
    uint32_t* stg = (uint32_t*)smem + wave * (64 * EPI_ROW);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if ((i / PB) & 1) continue;  // i is the low member; i + PB the high one
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = i * 32 + g * 8 + khalf * 4;  // feature offset in the wave (low member)
            const int nlo = min(nw + nl, N - 4), nhi = nlo + HALF;
            const int elo = nlo % D;
            const uint2 blo = *(const uint2*)(bias + nlo);
            const uint2 bhi = *(const uint2*)(bias + nhi);
            const float bl[4] = {bf16lo(blo.x), bf16hi(blo.x), bf16lo(blo.y), bf16hi(blo.y)};
            const float bh[4] = {bf16lo(bhi.x), bf16hi(bhi.x), bf16lo(bhi.y), bf16hi(bhi.y)};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int pl = j * 32 + (lane & 31);
                const int64_t p = min((int64_t)(pw + pl), T - 1);
                float ylo[4], yhi[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ylo[r] = acc[i][j][g * 4 + r] + bl[r];
                    yhi[r] = acc[i + PB][j][g * 4 + r] + bh[r];
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
    }
    __syncthreads();
    // 16 lanes per staged row, 16 bytes each: 4 full rows per store instruction.
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
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

#ifndef KVMAP_MAP_STAGES
#define KVMAP_MAP_STAGES 2
#endif

hipError_t launch_map_bf16(const MapArgs& a, const ApplyGeom& g, hipStream_t s) {
    const int N = g.N();
    const int nP = (int)((g.T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int grid = map_bf16_grid(g.L_tgt, g.T, N);
    constexpr int NS = KVMAP_MAP_STAGES;
    if (g.d == 128)
        hipLaunchKernelGGL((map_bf16_kernel<128, NS>), dim3(grid), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    else
        hipLaunchKernelGGL((map_bf16_kernel<64, NS>), dim3(grid), dim3(512), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    return hipGetLastError();
}

}  // namespace kvmap
