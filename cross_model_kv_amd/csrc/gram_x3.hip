// Co-moments of bf16 batches on the bf16 matrix cores (fit side, KVBridge README fitting
// section "Loading": centered covariance accumulated batchwise with the Chan/Welford update).
//
// For bf16 inputs the batch is shifted by c = its column means rounded to bf16 (a batch into
// an empty state) or the running mean rounded to bf16 (a merging batch, so the batch is read
// once), so that d = x - c is a difference of two bf16 values: exact in fp32 and, whenever the two are
// within a factor 2^7 of each other, exactly the sum hi + lo of two bf16 values
// (hi = bf16(d), lo = bf16(d - hi)); otherwise hi + lo carries d's leading 16 bits.  The
// products of the shifted data then come from three bf16 MFMA passes,
//   d_i d_j  =  hi_i hi_j + hi_i lo_j + lo_i hi_j   (+ lo_i lo_j, below 2^-16 of it, dropped)
// each product exact in the fp32 accumulator.
//
//   1. gram_split_kernel: per operand (X, then Y) and 32-token block, d, hi and lo, written
//      transposed as S [column][token block][hi of 32 tokens | lo of 32 tokens] (one
//      128-byte line per column and block), plus partial column sums of d (the small mean
//      of the shifted batch).
//   2. gram_x3_kernel: the upper triangle of 256 x 256 tiles of S_x S_x^T (or, for a state
//      that keeps M_xx block-diagonal, of each diagonal block) and all tiles of S_x S_y^T,
//      K = tokens, with the map GEMM's direct-to-LDS pipeline; the epilogue turns co-moments
//      about c into co-moments about the batch mean and merges them into the running state
//      (M += G - n_b m m^T + coef delta delta^T), writing off-diagonal tiles of M_xx to both
//      triangles.

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

namespace kvmap {

namespace {

constexpr int SP_COLS = 256;  // columns per split workgroup
constexpr int SP_TOK = 32;    // tokens per block (one K-step of the co-moment GEMM)
constexpr int SP_LD = SP_TOK + 1;

constexpr int GB = 256;        // co-moment tile (features x features)
constexpr int GSTAGE = GB * 8;  // 16-byte chunks per operand per K-step (2048)

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_f32(uint32_t h) { return __uint_as_float(h << 16); }

}  // namespace

// ---- 1: shift, split, transpose -------------------------------------------------------
// Workgroup: 256 columns; it walks token blocks blockIdx.y, + gridDim.y, ...  A thread reads
// 8 adjacent columns of 4 rows per block (one 16-byte load per row when the rows are 16-byte
// aligned, else two 8-byte halves), and holds the next block's rows in registers while the
// current one goes through LDS as (hi | lo << 16) per (column, token) and leaves as whole
// 128-byte lines, 8 lanes per line.  The column sums are reduced through the same LDS.
template <bool V16>
__global__ __launch_bounds__(256) void gram_split_kernel(const uint16_t* __restrict__ A, int64_t n_b, int cols,
                                                         int nkb, const float* __restrict__ c, int round_c,
                                                         uint16_t* __restrict__ S, float* __restrict__ part,
                                                         int part_stride, int col_off, float* __restrict__ part2) {
    __shared__ uint32_t t[SP_COLS * SP_LD];
    static_assert(2 * 8 * SP_COLS <= SP_COLS * SP_LD, "the column-sum reduction reuses the transpose buffer");
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * SP_COLS;
    const int rc = (tid & 31) * 8;  // first of the thread's 8 columns within the workgroup
    const int rr = tid >> 5;        // row within each group of 8
    // cols is a multiple of 4: each half (4 columns) of the thread's 8 is wholly in or out
    const bool cok0 = c0 + rc < cols, cok1 = c0 + rc + 4 < cols;
    float sh[8], sum[8], sum2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sh[e] = (e < 4 ? cok0 : cok1) ? c[c0 + rc + e] : 0.f;
        if (round_c) sh[e] = bf16_bits_f32(bf16_rne_bits(sh[e]));
        sum[e] = 0.f;
        sum2[e] = 0.f;
    }
    // rows tok = 8 pass + rr of block kb, 8 columns each as 4 words.  The loads themselves are
    // unconditional (rows past the batch and columns past the matrix read a valid element), so
    // the wait before a block's words are used counts only the loads of the block after it;
    // what lies outside the batch is zeroed when it is used.
    const int cl0 = cok0 ? c0 + rc : 0, cl1 = cok1 ? c0 + rc + 4 : 0;
    auto load = [&](int kb, uint32_t (&w)[4][4]) {
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int64_t row = std::min<int64_t>((int64_t)kb * SP_TOK + pass * 8 + rr, n_b - 1);
            if (V16) {
                const uint4 v = *(const uint4*)(A + row * cols + cl0);
                w[pass][0] = v.x;
                w[pass][1] = v.y;
                w[pass][2] = v.z;
                w[pass][3] = v.w;
            } else {
                const uint2 h0 = *(const uint2*)(A + row * cols + cl0);
                const uint2 h1 = *(const uint2*)(A + row * cols + cl1);
                w[pass][0] = h0.x;
                w[pass][1] = h0.y;
                w[pass][2] = h1.x;
                w[pass][3] = h1.y;
            }
        }
    };
    // LDS hand-off between the phases of a block: a plain barrier after this wave's LDS
    // operations (__syncthreads would also wait for the prefetched global loads)
    auto lds_sync = [&]() {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // one block through LDS to the split operand
    auto process = [&](int kb, const uint32_t (&w)[4][4]) {
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int tok = pass * 8 + rr;
            const bool inb = (int64_t)kb * SP_TOK + tok < n_b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t bits = (w[pass][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                const float d = ((e < 4 ? cok0 : cok1) && inb) ? bf16_bits_f32(bits) - sh[e] : 0.f;  // exact
                sum[e] += d;
                sum2[e] += d * d;
                const uint32_t hi = bf16_rne_bits(d);
                const uint32_t lo = bf16_rne_bits(d - bf16_bits_f32(hi));
                t[(rc + e) * SP_LD + tok] = hi | (lo << 16);
            }
        }
        lds_sync();
        // line (column, block): chunk ch < 4 = hi of tokens 8ch .. 8ch+7, ch >= 4 = lo of them
        const int ch = tid & 7;
        const int t0 = (ch & 3) * 8;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int col = (tid >> 3) + 32 * u;
            if (c0 + col < cols) {
                uint32_t o[4];
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    const uint32_t a = t[col * SP_LD + t0 + 2 * k2], b = t[col * SP_LD + t0 + 2 * k2 + 1];
                    o[k2] = ch >= 4 ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
                }
                *(uint4*)(S + ((size_t)(c0 + col) * nkb + kb) * 64 + ch * 8) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        lds_sync();
    };
    // Blocks in pairs of register buffers: the next block's loads (unconditional, a clamped
    // block past the end repeats the last one) are in flight while the current one is processed.
    uint32_t wa[4][4], wb[4][4];
    const int g = gridDim.y;
    int kb = blockIdx.y;
    load(kb, wa);
    while (true) {
        load(min(kb + g, nkb - 1), wb);
        process(kb, wa);
        kb += g;
        if (kb >= nkb) break;
        load(min(kb + g, nkb - 1), wa);
        process(kb, wb);
        kb += g;
        if (kb >= nkb) break;
    }
    float* red = (float*)t;  // [8][SP_COLS] sums, then [8][SP_COLS] sums of squares
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        red[rr * SP_COLS + rc + e] = sum[e];
        red[(8 + rr) * SP_COLS + rc + e] = sum2[e];
    }
    __syncthreads();
    if (c0 + tid < cols) {
        float s = 0.f, s2 = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            s += red[g * SP_COLS + tid];
            s2 += red[(8 + g) * SP_COLS + tid];
        }
        part[(size_t)blockIdx.y * part_stride + col_off + c0 + tid] = s;
        if (part2) part2[(size_t)blockIdx.y * part_stride + col_off + c0 + tid] = s2;
    }
}

namespace {

__device__ __forceinline__ void tri_decode256(int u, int nT, int& I, int& J) {
    // upper triangle (I <= J), row-major: row I starts at I*nT - I*(I-1)/2
    const double b = 2.0 * nT + 1.0;
    int i = (int)((b - sqrt(b * b - 8.0 * (double)u)) * 0.5);
    if (i < 0) i = 0;
    while (i > 0 && (int64_t)i * nT - (int64_t)i * (i - 1) / 2 > u) --i;
    while ((int64_t)(i + 1) * nT - (int64_t)(i + 1) * i / 2 <= u) ++i;
    I = i;
    J = i + (u - (int)((int64_t)i * nT - (int64_t)i * (i - 1) / 2));
}

}  // namespace

// ---- 2: co-moment GEMM on the split operands ------------------------------------------
// The map GEMM's pipeline with the roles A = S_x rows i (2-deep ring, loaded after the
// barrier) and B = S_x or S_y rows j (3-deep ring, loaded in the first substep of the next
// K-step), K-steps of 32 tokens = one 128-byte line (hi | lo) per row.  8 waves, wave w
// owns rows i (w & 1) * 128 .. + 127 and columns j (w >> 1) * 64 .. + 63 of the tile, as
// 8 x 4 blocks of v_mfma_f32_16x16x32_bf16 (16 x 16, 32 tokens deep).  A K-step:
//   first substep (8 chunks, one per A block i): hi_i hi_j and hi_i lo_j for the 4 B
//     blocks; the reads of lo_i for the second substep; the 4 B loads of K-step kb+2.
//   wait + barrier (K-step kb+1 landed everywhere, every read of K-step kb done).
//   second substep (4 chunks, one per B block j): lo_i hi_j for the 8 A blocks; then the
//     reads of K-step kb+1's hi_j (into the registers just freed), lo_j and two hi_i;
//     the 4 A loads of K-step kb+2.
__global__ __launch_bounds__(512) void gram_x3_kernel(const uint16_t* __restrict__ Sx,
                                                      const uint16_t* __restrict__ Sy, int nkb, int p,
                                                      int q, int nTx, int nXX, const float* __restrict__ mx,
                                                      const float* __restrict__ my,
                                                      const float* __restrict__ dx,
                                                      const float* __restrict__ dy, float coef, float nbf,
                                                      int fresh, float* __restrict__ M_xx,
                                                      float* __restrict__ M_xy, int bd, int nTb) {
    constexpr int NW = 8, LPO = 4, TW = 64, JB = 4, IB = 8;
    constexpr int TILE = GSTAGE * 16;  // 32 KB
    constexpr int NA = 2, NB = 3;
    __shared__ __attribute__((aligned(16))) char smem[(NA + NB) * TILE];
    uint4* lds = (uint4*)smem;

    // bd > 0: M_xx is kept as p / bd diagonal blocks of bd x bd (compact); blk is the block,
    // I, J count tiles from the matrix origin, b0 is the block's first feature
    int I, J, blk = 0;
    bool xy;
    if ((int)blockIdx.x < nXX) {
        if (bd) {
            const int per = nTb * (nTb + 1) / 2;
            blk = (int)blockIdx.x / per;
            tri_decode256((int)blockIdx.x - blk * per, nTb, I, J);
        } else {
            tri_decode256(blockIdx.x, nTx, I, J);
        }
        xy = false;
    } else {
        const int u = blockIdx.x - nXX;
        I = u % nTx;
        J = u / nTx;
        xy = true;
    }
    const int b0 = blk * bd;  // 0 unless blocked
    const int i0 = b0 + I * GB, j0 = b0 + J * GB;
    const int ldb = xy ? q : p;
    const uint16_t* __restrict__ Bs = xy ? Sy : Sx;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t row_bytes = (uint32_t)nkb * 128u;
    const i32x4_t ar = make_rsrc(Sx + (size_t)i0 * nkb * 64, row_bytes * GB);
    const i32x4_t br = make_rsrc(Bs + (size_t)j0 * nkb * 64, row_bytes * GB);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);

    // Loads: LDS slot u = i*512 + wave*64 + lane of a tile buffer holds row u/8, chunk
    // (u%8) ^ slot_xor(row); rows past the matrix repeat its last row (never stored).
    int aoff[LPO], boff[LPO];
#pragma unroll
    for (int i = 0; i < LPO; ++i) {
        const int r = i * 8 * NW + wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ slot_xor(r);
        const int ra = min(r, p - 1 - i0), rb = min(r, ldb - 1 - j0);
        aoff[i] = (int)((uint32_t)ra * row_bytes) + c * 16;
        boff[i] = (int)((uint32_t)rb * row_bytes) + c * 16;
    }
    const int k_last = (nkb - 1) * 128;
    int a_buf = 0, a_soff = 0, b_buf = 0, b_soff = 0;
    struct Issue {
        uint32_t la;
        int soff;
    };
    auto plan_a = [&]() {
        const Issue r = {lds_base + (uint32_t)a_buf * TILE + wave_s * 1024u, a_soff};
        a_buf = (a_buf + 1 == NA) ? 0 : a_buf + 1;
        a_soff = min(a_soff + 128, k_last);
        return r;
    };
    auto plan_b = [&]() {
        const Issue r = {lds_base + (uint32_t)(NA + b_buf) * TILE + wave_s * 1024u, b_soff};
        b_buf = (b_buf + 1 == NB) ? 0 : b_buf + 1;
        b_soff = min(b_soff + 128, k_last);
        return r;
    };
    auto issue_a1 = [&](const Issue& r, int i) { lds_dma16(ar, r.la + i * 1024 * NW, aoff[i], r.soff); };
    auto issue_b1 = [&](const Issue& r, int i) { lds_dma16(br, r.la + i * 1024 * NW, boff[i], r.soff); };

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
    // Fragment of half h (0 = hi, 1 = lo) of a K-step: lane holds row (lane % 16) + 16 i of
    // its block, tokens 8 (lane / 16) .. + 7 of the 32.
    auto rd_a = [&](int buf, int h, int i) {
        return __builtin_bit_cast(bf16x8_t, lds[buf * GSTAGE + arow + i * 128 + ((h * 4 + kq) ^ fx)]);
    };
    auto rd_b = [&](int buf, int h, int j) {
        return __builtin_bit_cast(bf16x8_t, lds[(NA + buf) * GSTAGE + brow + j * 128 + ((h * 4 + kq) ^ fx)]);
    };
    auto sync = [&]() {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // prologue: A(0) B(0) A(1) B(1); K-step 0 is complete once only A(1) B(1) remain
    {
        const Issue a0 = plan_a(), b0 = plan_b(), a1 = plan_a(), b1 = plan_b();
#pragma unroll
        for (int i = 0; i < LPO; ++i) issue_a1(a0, i);
#pragma unroll
        for (int i = 0; i < LPO; ++i) issue_b1(b0, i);
#pragma unroll
        for (int i = 0; i < LPO; ++i) issue_a1(a1, i);
#pragma unroll
        for (int i = 0; i < LPO; ++i) issue_b1(b1, i);
    }
    Issue b_next = plan_b();  // B(2), issued during K-step 0
    Issue a_next;             // A(kb+2), planned during K-step kb
    bf16x8_t ahi[IB], alo[IB], bhi[JB], blo[JB];
    wait_vmcnt<2 * LPO>();
    sync();
    int ca = 0, cb = 0;
#pragma unroll
    for (int i = 0; i < IB; ++i) ahi[i] = rd_a(ca, 0, i);
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        bhi[j] = rd_b(cb, 0, j);
        blo[j] = rd_b(cb, 1, j);
    }
    auto kstep = [&]() {  // one K-step
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            alo[i] = rd_a(ca, 1, i);
#pragma unroll
            for (int j = 0; j < JB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[i], bhi[j], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < JB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[i], blo[j], acc[i][j], 0, 0, 0);
            if (i & 1) issue_b1(b_next, i >> 1);  // B(kb+2) -> B buffer of K-step kb-1
            if (i == 2) a_next = plan_a();
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<LPO>();
        sync();
        const int ca1 = (ca + 1 == NA) ? 0 : ca + 1;
        const int cb1 = (cb + 1 == NB) ? 0 : cb + 1;
        // (after the last K-step this reads buffers that are never used)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            issue_a1(a_next, j);  // A(kb+2) -> A buffer of K-step kb
#pragma unroll
            for (int i = 0; i < IB; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[i], bhi[j], acc[i][j], 0, 0, 0);
            bhi[j] = rd_b(cb1, 0, j);
            blo[j] = rd_b(cb1, 1, j);
            ahi[2 * j] = rd_a(ca1, 0, 2 * j);
            ahi[2 * j + 1] = rd_a(ca1, 0, 2 * j + 1);
            if (j == 1) b_next = plan_b();
            __builtin_amdgcn_sched_barrier(0);
        }
        ca = ca1;
        cb = cb1;
    };
    // two K-steps per trip of the loop, as in the map GEMM; an odd count ends with one more
    int kb = 0;
    for (; kb + 2 <= nkb; kb += 2) {
        kstep();
        kstep();
    }
    if (kb < nkb) kstep();
    wait_vmcnt<0>();

    // Epilogue: lane holds G[i][j] for j = column (lane & 15) and i = 4 (lane / 16) + r of
    // each 16 x 16 block.
    // M_xx of a blocked state: block blk at M_xx + blk bd^2, local row/column, leading dim bd
    const bool blocked = !xy && bd;
    float* __restrict__ M = xy ? M_xy : (blocked ? M_xx + (size_t)blk * bd * bd : M_xx);
    const int ldm = xy ? q : (blocked ? bd : p);
    const int moff = blocked ? b0 : 0;
    const int lim = blocked ? b0 + bd : p;  // rows and columns of M_xx's block (or of M_xx)
    const float* __restrict__ mb = xy ? my : mx;
    const float* __restrict__ db = xy ? dy : dx;
    const bool mirror = !xy && I != J;
    // Per 16-column block and half of the row blocks: every old value of the state is read
    // before any store of the group (as load-add-store element by element, each load would
    // wait for the previous store).
    constexpr int IH = IB / 2;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
        const int j = j0 + wp * TW + jb * 16 + (lane & 15);
        const bool jok = j < (xy ? ldb : lim);
        const float mj = jok ? mb[j] : 0.f, dj = jok ? db[j] : 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float old[IH][4], oldm[IH][4];
#pragma unroll
            for (int u = 0; u < IH; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) old[u][r] = oldm[u][r] = 0.f;
            if (!fresh) {
#pragma unroll
                for (int u = 0; u < IH; ++u) {
                    const int i = i0 + wn * 128 + (h * IH + u) * 16 + kq * 4;
                    if (!jok || i >= lim) continue;  // p and bd are multiples of 4: all 4 rows valid
#pragma unroll
                    for (int r = 0; r < 4; ++r) old[u][r] = M[(size_t)(i - moff + r) * ldm + (j - moff)];
                    if (mirror) {
                        const float4 o = *(const float4*)(M + (size_t)(j - moff) * ldm + (i - moff));
                        oldm[u][0] = o.x;
                        oldm[u][1] = o.y;
                        oldm[u][2] = o.z;
                        oldm[u][3] = o.w;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < IH; ++u) {
                const int ib = h * IH + u;
                const int i = i0 + wn * 128 + ib * 16 + kq * 4;
                if (!jok || i >= lim) continue;
                const float4 mi = *(const float4*)(mx + i);
                const float4 di = *(const float4*)(dx + i);
                const float mia[4] = {mi.x, mi.y, mi.z, mi.w};
                const float dia[4] = {di.x, di.y, di.z, di.w};
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[ib][jb][r] - nbf * mia[r] * mj + coef * dia[r] * dj;
#pragma unroll
                for (int r = 0; r < 4; ++r) M[(size_t)(i - moff + r) * ldm + (j - moff)] = old[u][r] + v[r];
                if (mirror)
                    *(float4*)(M + (size_t)(j - moff) * ldm + (i - moff)) =
                        make_float4(oldm[u][0] + v[0], oldm[u][1] + v[1], oldm[u][2] + v[2], oldm[u][3] + v[3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------

size_t gram_split_elems(int p, int q, int64_t n_b) {
    const int64_t nkb = (n_b + SP_TOK - 1) / SP_TOK;
    return (size_t)(p + q) * (size_t)nkb * 64;
}

int gram_split_blocks(int64_t n_b, int max_splits) {
    const int64_t nkb = (n_b + SP_TOK - 1) / SP_TOK;
    return (int)std::min<int64_t>(nkb, max_splits);
}

hipError_t launch_gram_split(const void* A, int64_t n_b, int cols, const float* c, int round_c, uint16_t* S,
                             float* part, int part_stride, int col_off, float* part2, int splits, hipStream_t s) {
    const int nkb = (int)((n_b + SP_TOK - 1) / SP_TOK);
    const dim3 grid((cols + SP_COLS - 1) / SP_COLS, splits);
    // 16-byte row loads when every row starts 16-byte aligned (A itself is)
    if (cols % 8 == 0 && ((uintptr_t)A & 15) == 0)
        hipLaunchKernelGGL(gram_split_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)A, n_b, cols, nkb, c,
                           round_c, S, part, part_stride, col_off, part2);
    else
        hipLaunchKernelGGL(gram_split_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)A, n_b, cols, nkb, c,
                           round_c, S, part, part_stride, col_off, part2);
    return hipGetLastError();
}

hipError_t launch_gram_x3(const uint16_t* Sx, const uint16_t* Sy, int64_t n_b, int p, int q, const float* mx,
                          const float* my, const float* dx, const float* dy, float coef, int fresh,
                          float* M_xx, float* M_xy, int bd, hipStream_t s) {
    const int nkb = (int)((n_b + SP_TOK - 1) / SP_TOK);
    const int nTx = (p + GB - 1) / GB, nTy = (q + GB - 1) / GB;
    const int nTb = bd ? (bd + GB - 1) / GB : 0;
    const int nXX = bd ? (p / bd) * (nTb * (nTb + 1) / 2) : nTx * (nTx + 1) / 2;
    const int blocks = nXX + nTx * nTy;
    hipLaunchKernelGGL(gram_x3_kernel, dim3(blocks), dim3(512), 0, s, Sx, Sy, nkb, p, q, nTx, nXX, mx, my, dx,
                       dy, coef, (float)n_b, fresh, M_xx, M_xy, bd, nTb);
    return hipGetLastError();
}

}  // namespace kvmap
