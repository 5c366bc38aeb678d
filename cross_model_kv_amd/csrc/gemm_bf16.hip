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
constexpr int BK = 64;   // features (reduction) per K-step
constexpr int CHUNKS = BM * BK / 8;  // 16-byte chunks per operand tile (2048)

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

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

}  // namespace

int map_bf16_grid(int L_tgt, int64_t T, int N) {
    const int nP = (int)((T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int pg = nN >= 32 ? 1 : 32 / nN;
    const int spk = (nP + pg - 1) / pg;
    const int S = L_tgt * 2 * spk;
    return ((S + 7) / 8) * pg * nN * 8;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [base, base + bytes) for raw buffer loads (gfx9 dword3 = 0x00020000).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One K-step of the main loop on LDS buffers (curA, curB), with the next K-step's tiles
// streamed straight from HBM into (nxtA, nxtB) by buffer_load_dwordx4 ... lds (no staging
// registers, no ds_write).  LDS slot u of a tile holds the 16-byte chunk (row u/8,
// column (u%8) ^ (row&7)): wave w's i-th load fills slots i*256 + w*64 + lane.  Per-lane
// byte offsets are fixed for the whole K loop; the K-step moves only scalar state (the W
// soffset and the gathered slab's resource base).
#define KVMAP_STEP(kt, curA, curB, nxtA, nxtB)                                              \
    do {                                                                                    \
        if ((kt) + 1 < nk) {                                                                \
            const int k1 = ((kt) + 1) * BK;                                                 \
            const int s1 = k1 / D, e1 = k1 - s1 * D;                                        \
            const int j1 = s1 / H, h1 = s1 - j1 * H;                                        \
            const __amdgpu_buffer_rsrc_t xr =                                               \
                make_rsrc(X + ((size_t)sel[j1] * H + h1) * slab + e1, slab_bytes);          \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                 \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(                                   \
                    wr, (lds_ptr_t)((nxtA) + i * 256 + wave * 64), 16, aoff[i], k1 * 2, 0, 0); \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(                                   \
                    xr, (lds_ptr_t)((nxtB) + i * 256 + wave * 64), 16, boff[i], 0, 0, 0);   \
            }                                                                               \
        }                                                                                   \
        _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks) {                            \
            const int ch = ks * 2 + khalf;                                                  \
            bf16x8_t fa[4], fb[4];                                                          \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                 \
                fa[i] = __builtin_bit_cast(bf16x8_t, (curA)[swz(arow0 + 32 * i, ch)]);      \
                fb[i] = __builtin_bit_cast(bf16x8_t, (curB)[swz(brow0 + 32 * i, ch)]);      \
            }                                                                               \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                   \
                _Pragma("unroll") for (int j = 0; j < 4; ++j)                               \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j],       \
                                                                        acc[i][j], 0, 0, 0); \
        }                                                                                   \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                    \
        __syncthreads();                                                                    \
    } while (0)

template <int D>
__global__ __launch_bounds__(256, 1) void map_bf16_kernel(MapArgs a, int L_tgt, int H, int k,
                                                          int64_t T, int nP, int nN) {
    __shared__ uint4 ldsA0[CHUNKS], ldsB0[CHUNKS], ldsA1[CHUNKS], ldsB1[CHUNKS];

    TileId tl;
    if (!decode_tile(blockIdx.x, L_tgt, nP, nN, tl)) return;

    const int N = H * D, F = k * N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = tl.nb * BM, p0 = tl.pb * BN;
    const uint16_t* __restrict__ X = (const uint16_t*)(tl.kv ? a.xv : a.xk);
    const uint16_t* __restrict__ W = (const uint16_t*)(tl.kv ? a.Wv : a.Wk) + (size_t)tl.t * N * F;
    const int32_t* __restrict__ sel = a.sel + tl.t * k;
    const size_t slab = (size_t)T * D;

    // Byte offsets (within a K-step) of the chunks this lane streams into LDS.
    int aoff[8], boff[8];
    {
        const int r8 = lane >> 3;
        const int col = (lane & 7) ^ (r8 & 7);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = i * 32 + wave * 8 + r8;
            const int n = min(n0 + r, N - 1);
            const int64_t p = min((int64_t)(p0 + r), T - 1);
            aoff[i] = (n * F + col * 8) * 2;
            boff[i] = ((int)(p * D) + col * 8) * 2;
        }
    }
    const uint32_t slab_bytes = (uint32_t)(slab * 2);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)((size_t)N * F * 2));

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int wn = wave & 1, wp = wave >> 1;
    const int arow0 = wn * 128 + (lane & 31);
    const int brow0 = wp * 128 + (lane & 31);
    const int khalf = lane >> 5;
    const int nk = F / BK;

    // prologue: K-step 0 into buffer 0
    {
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (size_t)sel[0] * H * slab, slab_bytes);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(ldsA0 + i * 256 + wave * 64), 16, aoff[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(ldsB0 + i * 256 + wave * 64), 16, boff[i], 0, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
        KVMAP_STEP(kt, ldsA0, ldsB0, ldsA1, ldsB1);
        KVMAP_STEP(kt + 1, ldsA1, ldsB1, ldsA0, ldsB0);
    }
    if (kt < nk) KVMAP_STEP(kt, ldsA0, ldsB0, ldsA1, ldsB1);  // odd number of K-steps

    // ---- epilogue: + bias, target RoPE on keys, bf16 store into [t][h][p][e] ----
    // Lane holds D[n][p] for p = col (lane & 31) and n = 8*(r/4) + 4*(lane/32) + r%4 of each
    // 32x32 block: 4 consecutive features per register group -> one 8-byte store.
    constexpr int HALF = D / 2;
    constexpr int PB = HALF / 32;  // block distance between the two members of a pair
    const uint16_t* __restrict__ bias = (const uint16_t*)(tl.kv ? a.bv : a.bk) + (size_t)tl.t * N;
    uint16_t* __restrict__ out = (uint16_t*)(tl.kv ? a.outv : a.outk);
    const int nw = n0 + wn * 128;
    const bool rope = (tl.kv == 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if ((i / PB) & 1) continue;  // i is the low member; i + PB the high one
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = i * 32 + g * 8 + khalf * 4;          // feature offset in wave
            const int nlo = nw + nl, nhi = nlo + HALF;
            if (nlo >= N) continue;
            const int h = nlo / D, elo = nlo - h * D;
            const uint2 blo = *(const uint2*)(bias + nlo);
            const uint2 bhi = *(const uint2*)(bias + nhi);
            const float bl[4] = {bf16lo(blo.x), bf16hi(blo.x), bf16lo(blo.y), bf16hi(blo.y)};
            const float bh[4] = {bf16lo(bhi.x), bf16hi(bhi.x), bf16lo(bhi.y), bf16hi(bhi.y)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t p = p0 + wp * 128 + j * 32 + (lane & 31);
                if (p >= T) continue;
                float ylo[4], yhi[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ylo[r] = acc[i][j][g * 4 + r] + bl[r];
                    yhi[r] = acc[i + PB][j][g * 4 + r] + bh[r];
                }
                if (rope) {
                    const float4* cs = (const float4*)(a.tab_tgt + p * HALF + elo);
                    const float4 c01 = cs[0], c23 = cs[1];
                    const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
                    const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float l = ylo[r], hh = yhi[r];
                        ylo[r] = fmaf(-hh, ss[r], l * cc[r]);
                        yhi[r] = fmaf(l, ss[r], hh * cc[r]);
                    }
                }
                uint16_t* o = out + (((size_t)tl.t * H + h) * T + p) * D + elo;
                *(uint2*)o = make_uint2(pack_bf16(ylo[0], ylo[1]), pack_bf16(ylo[2], ylo[3]));
                *(uint2*)(o + HALF) = make_uint2(pack_bf16(yhi[0], yhi[1]), pack_bf16(yhi[2], yhi[3]));
            }
        }
    }
}

hipError_t launch_map_bf16(const MapArgs& a, const ApplyGeom& g, hipStream_t s) {
    const int N = g.N();
    const int nP = (int)((g.T + BN - 1) / BN), nN = (N + BM - 1) / BM;
    const int grid = map_bf16_grid(g.L_tgt, g.T, N);
    if (g.d == 128)
        hipLaunchKernelGGL(map_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    else
        hipLaunchKernelGGL(map_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a, g.L_tgt, g.H, g.k, g.T, nP, nN);
    return hipGetLastError();
}

}  // namespace kvmap
