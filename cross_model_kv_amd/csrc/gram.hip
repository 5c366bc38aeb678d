// Fit-side statistics: centered co-moments of a batch, merged into a running state with
// the Chan/Welford pairwise update (KVBridge README, fitting section headed "Loading": the
// statistics stay centered batch by batch, so no large raw moments are ever subtracted).
//
// Per batch of n_b rows (x in R^p, y in R^q):
//   1. column sums (wavefront/LDS reduced)  -> shift c = fp32 column mean
//   2. column sums of (x - c)               -> m = mean of the shifted batch (tiny)
//      batch mean = c + m;  delta = batch mean - running mean;  running mean updated
//   3. co-moments on the matrix cores in fp32 (v_mfma_f32_32x32x2_f32) of the shifted data
//        G = sum (x - c)(x - c)^T,  C = sum (x - c)(y - c_y)^T
//      fused with the merge in the epilogue:
//        M_xx += G - n_b m m^T + (n n_b / n') delta delta^T       (n' = n + n_b)
//   The shift makes every product small (the inputs carry offsets ~5 in the fit-stat
//   workload), so nothing cancels; the rank-one n_b m m^T term turns the co-moments about c
//   into co-moments about the exact batch mean.  Only the upper triangle of tiles of M_xx
//   is computed; off-diagonal tiles are written to both triangles.

#include "common.h"
#include "internal.h"

namespace kvmap {

namespace {
constexpr int CS_THREADS = 256;
constexpr int CS_COLS = 4;                       // columns per lane
constexpr int CS_TILE = 64 * CS_COLS;            // columns per workgroup (one wave wide)
constexpr int GT = 128;                          // Gram tile (features x features)
constexpr int GK = 32;                           // rows per K-step
constexpr int GLD = GT + 32;                     // padded LDS row (floats)
}  // namespace

size_t gram_scratch_floats(int p, int q, int splits) {
    return 2 * (size_t)splits * (p + q) + 3 * (size_t)(p + q);  // part, part2, c, m, delta
}

// ---- 1/2: column sums ---------------------------------------------------------------
// Lane owns 4 adjacent columns; the 4 waves of a workgroup take interleaved rows of the
// workgroup's row split and are reduced through LDS; splits are reduced by the finalize
// kernel in a fixed order (deterministic, no atomics).
template <bool BF16>
__global__ __launch_bounds__(CS_THREADS) void colsum_kernel(const void* __restrict__ A,
                                                            int64_t n, int cols,
                                                            const float* __restrict__ shift,
                                                            float* __restrict__ part,
                                                            int part_stride, int col_off,
                                                            float* __restrict__ part2) {
    __shared__ float4 red[4][64];
    __shared__ float4 red2[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * CS_TILE + lane * CS_COLS;
    const int splits = gridDim.y;
    const int64_t r0 = n * blockIdx.y / splits, r1 = n * (blockIdx.y + 1) / splits;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), acc2 = acc;
    if (c0 < cols) {
        float4 sh = make_float4(0.f, 0.f, 0.f, 0.f);
        if (shift) sh = *(const float4*)(shift + c0);
        for (int64_t r = r0 + wave; r < r1; r += 4) {
            float4 v;
            if (BF16) {
                const uint2 w = *(const uint2*)((const uint16_t*)A + r * cols + c0);
                v = make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
            } else {
                v = *(const float4*)((const float*)A + r * cols + c0);
            }
            const float4 dv = make_float4(v.x - sh.x, v.y - sh.y, v.z - sh.z, v.w - sh.w);
            acc.x += dv.x; acc.y += dv.y; acc.z += dv.z; acc.w += dv.w;
            acc2.x += dv.x * dv.x; acc2.y += dv.y * dv.y; acc2.z += dv.z * dv.z; acc2.w += dv.w * dv.w;
        }
    }
    red[wave][lane] = acc;
    red2[wave][lane] = acc2;
    __syncthreads();
    if (wave == 0 && c0 < cols) {
        float4 s = red[0][lane], s2 = red2[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const float4 o = red[w][lane], o2 = red2[w][lane];
            s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
            s2.x += o2.x; s2.y += o2.y; s2.z += o2.z; s2.w += o2.w;
        }
        *(float4*)(part + (size_t)blockIdx.y * part_stride + col_off + c0) = s;
        if (part2) *(float4*)(part2 + (size_t)blockIdx.y * part_stride + col_off + c0) = s2;
    }
}

// sum_y part[y * stride + col] over y = 0 .. splits - 1 in float64, in that order; the loads go
// out 16 at a time (one dependent load per split had made the finalize latency-bound).
__device__ __forceinline__ double sum_splits(const float* __restrict__ part, int splits, int stride, int col) {
    double s = 0.0;
    int y = 0;
    for (; y + 16 <= splits; y += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = part[(size_t)(y + u) * stride + col];
#pragma unroll
        for (int u = 0; u < 16; ++u) s += (double)v[u];
    }
    for (; y < splits; ++y) s += (double)part[(size_t)y * stride + col];
    return s;
}

// Reduce the split partial sums (float64, fixed order) and derive the phase's outputs.
//   phase 0: c = sum / n_b (rounded to bf16 when round_c: the split co-moment path shifts
//            bf16 data by a bf16 value, so that x - c is exact)
//   phase 1: m = sum / n_b; batch mean = c + m; delta = batch mean - mean; mean updated;
//            with round_c the shift c was not stored but is the running mean rounded to bf16
//            (the split path of a merging call), formed here again before the mean moves;
//            with ss_y (and the partial sums of squares of the shifted y in part2): the
//            centered sum of squares of y merged the same way (Chan):
//            ss_y += (sum2 - n_b m^2) + n n_b / n' delta^2
__global__ __launch_bounds__(256) void colsum_finalize_kernel(
    const float* __restrict__ part, int splits, int p, int q, int64_t n_b, int64_t n_old,
    int phase, int round_c, float* __restrict__ cx, float* __restrict__ cy, float* __restrict__ mx,
    float* __restrict__ my, float* __restrict__ dx, float* __restrict__ dy,
    float* __restrict__ mean_x, float* __restrict__ mean_y, const float* __restrict__ part2,
    float* __restrict__ ss_y) {
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    const int stride = p + q;
    if (col >= stride) return;
    const double s = sum_splits(part, splits, stride, col);
    const double mean_b = s / (double)n_b;
    const bool isx = col < p;
    const int c = isx ? col : col - p;
    float* cc = isx ? cx : cy;
    if (phase == 0) {
        float cf = (float)mean_b;
        if (round_c) {
            uint32_t u = __float_as_uint(cf);
            u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even, to bf16
            cf = __uint_as_float(u & 0xffff0000u);
        }
        cc[c] = cf;
        return;
    }
    float* mm = isx ? mx : my;
    float* dd = isx ? dx : dy;
    float* mean = isx ? mean_x : mean_y;
    mm[c] = (float)mean_b;
    double shift = (double)cc[c];
    if (round_c) {
        uint32_t u = __float_as_uint(mean[c]);
        u += 0x7fffu + ((u >> 16) & 1u);
        shift = (double)__uint_as_float(u & 0xffff0000u);
    }
    const double bm = shift + mean_b;
    double delta = 0.0;
    if (n_old == 0) {
        dd[c] = 0.f;
        mean[c] = (float)bm;
    } else {
        const double old = (double)mean[c];
        delta = bm - old;
        dd[c] = (float)delta;
        mean[c] = (float)(old + delta * ((double)n_b / (double)(n_old + n_b)));
    }
    if (!isx && ss_y) {
        const double s2 = sum_splits(part2, splits, stride, col);
        const double ssb = s2 - (double)n_b * mean_b * mean_b;
        const double coef = (double)n_old * (double)n_b / (double)(n_old + n_b);
        ss_y[c] = (float)((n_old == 0 ? 0.0 : (double)ss_y[c]) + ssb + coef * delta * delta);
    }
}

// ---- 3: shifted co-moments + merge ---------------------------------------------------
__device__ __forceinline__ void tri_decode(int u, int nT, int& I, int& J) {
    // upper triangle (I <= J), row-major: row I starts at I*nT - I*(I-1)/2
    const double b = 2.0 * nT + 1.0;
    int i = (int)((b - sqrt(b * b - 8.0 * (double)u)) * 0.5);
    if (i < 0) i = 0;
    while (i > 0 && (int64_t)i * nT - (int64_t)i * (i - 1) / 2 > u) --i;
    while ((int64_t)(i + 1) * nT - (int64_t)(i + 1) * i / 2 <= u) ++i;
    I = i;
    J = i + (u - (int)((int64_t)i * nT - (int64_t)i * (i - 1) / 2));
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* base, int64_t row, int64_t ld, int col) {
    if (BF16) {
        const uint2 w = *(const uint2*)((const uint16_t*)base + row * ld + col);
        return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
    }
    return *(const float4*)((const float*)base + row * ld + col);
}

template <bool BF16>
__global__ __launch_bounds__(256, 1) void gram_kernel(
    const void* __restrict__ X, const void* __restrict__ Y, int64_t n_b, int p, int q,
    const float* __restrict__ cx, const float* __restrict__ cy, const float* __restrict__ mx,
    const float* __restrict__ my, const float* __restrict__ dx, const float* __restrict__ dy,
    float coef, int fresh, float* __restrict__ M_xx, float* __restrict__ M_xy, int nTx, int nXX, int bd,
    int nTb) {
    __shared__ float4 lds[2][2][GK * GLD / 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // bd > 0: M_xx kept as p / bd compact diagonal blocks (see the bf16 co-moment kernel)
    int I, J, blk = 0;
    bool xy;
    if ((int)blockIdx.x < nXX) {
        if (bd) {
            const int per = nTb * (nTb + 1) / 2;
            blk = (int)blockIdx.x / per;
            tri_decode((int)blockIdx.x - blk * per, nTb, I, J);
        } else {
            tri_decode(blockIdx.x, nTx, I, J);
        }
        xy = false;
    } else {
        const int u = blockIdx.x - nXX;
        I = u % nTx;
        J = u / nTx;
        xy = true;
    }
    const int b0 = blk * bd;
    const int i0 = b0 + I * GT, j0 = b0 + J * GT;
    const void* B = xy ? Y : X;
    const int ldb = xy ? q : p;
    const float* cb = xy ? cy : cx;

    // Load mapping: chunk idx = tid + 256*u (u < 4): row = idx / 32, col = 4 * (idx % 32).
    const int lcol = (tid & 31) * 4;
    const int acol = min(i0 + lcol, p - 4), bcol = min(j0 + lcol, ldb - 4);
    const float4 sa = *(const float4*)(cx + acol);
    const float4 sb = *(const float4*)(cb + bcol);
    float4 ra[4], rb[4];
    auto gload = [&](int kt) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t row = (int64_t)kt * GK + (tid >> 5) + 8 * u;
            if (row < n_b) {
                float4 va = load4<BF16>(X, row, p, acol);
                float4 vb = load4<BF16>(B, row, ldb, bcol);
                ra[u] = make_float4(va.x - sa.x, va.y - sa.y, va.z - sa.z, va.w - sa.w);
                rb[u] = make_float4(vb.x - sb.x, vb.y - sb.y, vb.z - sb.z, vb.w - sb.w);
            } else {
                ra[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                rb[u] = ra[u];
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = (tid >> 5) + 8 * u;
            lds[buf][0][(row * GLD + lcol) / 4] = ra[u];
            lds[buf][1][(row * GLD + lcol) / 4] = rb[u];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int wi = wave & 1, wj = wave >> 1;
    const int nk = (int)((n_b + GK - 1) / GK);
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const float* As = (const float*)lds[buf][0];
        const float* Bs = (const float*)lds[buf][1];
#pragma unroll
        for (int ks = 0; ks < GK / 2; ++ks) {
            const int kr = (ks * 2 + (lane >> 5)) * GLD;
            float fa[2], fb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                fa[a] = As[kr + wi * 64 + a * 32 + (lane & 31)];
                fb[a] = Bs[kr + wj * 64 + a * 32 + (lane & 31)];
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds G[i][j] for column j = lane & 31 of each 32x32 block and rows
    // i = 8*(r/4) + 4*(lane/32) + r%4.
    const bool blocked = !xy && bd;
    float* M = xy ? M_xy : (blocked ? M_xx + (size_t)blk * bd * bd : M_xx);
    const int ldm = xy ? q : (blocked ? bd : p);
    const int moff = blocked ? b0 : 0;
    const int lim = xy ? q : (blocked ? b0 + bd : p);  // column limit
    const int rlim = blocked ? b0 + bd : p;            // row limit
    const float* mb = xy ? my : mx;
    const float* db = xy ? dy : dx;
    const float nbf = (float)n_b;
    const bool mirror = !xy && I != J;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int j = j0 + wj * 64 + b * 32 + (lane & 31);
        const bool jok = j < lim;
        const float mj = jok ? mb[j] : 0.f, dj = jok ? db[j] : 0.f;
        // per (column block, row half): the old values are read before any store of the group
        // (element-wise load-add-store would make each load wait for the previous store)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            float old[4][4], oldm[4][4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) old[g][r] = oldm[g][r] = 0.f;
            if (!fresh) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ib = i0 + wi * 64 + a * 32 + g * 8 + (lane >> 5) * 4;
                    if (ib >= rlim || !jok) continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r) old[g][r] = M[(size_t)(ib - moff + r) * ldm + (j - moff)];
                    if (mirror) {
                        const float4 o = *(const float4*)(M + (size_t)(j - moff) * ldm + (ib - moff));
                        oldm[g][0] = o.x; oldm[g][1] = o.y; oldm[g][2] = o.z; oldm[g][3] = o.w;
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ib = i0 + wi * 64 + a * 32 + g * 8 + (lane >> 5) * 4;
                if (ib >= rlim || !jok) continue;
                const float4 mi = *(const float4*)(mx + ib);
                const float4 di = *(const float4*)(dx + ib);
                float v[4];
                const float mia[4] = {mi.x, mi.y, mi.z, mi.w};
                const float dia[4] = {di.x, di.y, di.z, di.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] = acc[a][b][g * 4 + r] - nbf * mia[r] * mj + coef * dia[r] * dj;
#pragma unroll
                for (int r = 0; r < 4; ++r) M[(size_t)(ib - moff + r) * ldm + (j - moff)] = old[g][r] + v[r];
                if (mirror)
                    *(float4*)(M + (size_t)(j - moff) * ldm + (ib - moff)) =
                        make_float4(oldm[g][0] + v[0], oldm[g][1] + v[1], oldm[g][2] + v[2], oldm[g][3] + v[3]);
            }
        }
    }
}

hipError_t launch_gram_batch(Elem e, const void* X, const void* Y, int64_t n_b, int p, int q,
                             int64_t n_old, float* mean_x, float* mean_y, float* M_xx,
                             float* M_xy, float* ss_y, int bd, const GramScratch& sc, hipStream_t s) {
    const bool bf = (e == Elem::BF16);
    const dim3 gx((p + CS_TILE - 1) / CS_TILE, sc.splits), gy((q + CS_TILE - 1) / CS_TILE, sc.splits);
    const int stride = p + q;
    const unsigned fin = (unsigned)((stride + 255) / 256);
    const double n_new = (double)n_old + (double)n_b;
    const float coef = (float)((double)n_old * (double)n_b / n_new);
    const int fresh = (n_old == 0);
    if (bf) {
        // Shift c: a fresh state takes the batch's column means rounded to bf16 (one pass of
        // column sums first); a merging call takes the running mean rounded to bf16, which is
        // already on the device, so the batch is read once.  Either way x - c is exact and
        // the batch's own mean m of x - c is removed in the epilogue, so the shift only sets
        // how far the split values sit from the batch mean.  Then: split (d, hi, lo,
        // transposed) with the sums of d; m, delta, mean; co-moments on the bf16 matrix cores.
        const float* shx = sc.cx;
        const float* shy = sc.cy;
        if (fresh) {
            hipLaunchKernelGGL(colsum_kernel<true>, gx, dim3(CS_THREADS), 0, s, X, n_b, p, nullptr, sc.part, stride,
                               0, nullptr);
            hipLaunchKernelGGL(colsum_kernel<true>, gy, dim3(CS_THREADS), 0, s, Y, n_b, q, nullptr, sc.part, stride,
                               p, nullptr);
            hipLaunchKernelGGL(colsum_finalize_kernel, dim3(fin), dim3(256), 0, s, sc.part, sc.splits, p, q, n_b,
                               n_old, 0, 1, sc.cx, sc.cy, sc.mx, sc.my, sc.dx, sc.dy, mean_x, mean_y, nullptr,
                               nullptr);
        } else {
            shx = mean_x;
            shy = mean_y;
        }
        const int ss = gram_split_blocks(n_b, sc.max_splits);
        uint16_t* Sx = sc.split;
        uint16_t* Sy = sc.split + gram_split_elems(p, 0, n_b);
        hipError_t err = launch_gram_split(X, n_b, p, shx, !fresh, Sx, sc.part, stride, 0, nullptr, ss, s);
        if (err != hipSuccess) return err;
        err = launch_gram_split(Y, n_b, q, shy, !fresh, Sy, sc.part, stride, p, ss_y ? sc.part2 : nullptr, ss, s);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(colsum_finalize_kernel, dim3(fin), dim3(256), 0, s, sc.part, ss, p, q, n_b, n_old, 1,
                           fresh ? 0 : 1, sc.cx, sc.cy, sc.mx, sc.my, sc.dx, sc.dy, mean_x, mean_y, sc.part2, ss_y);
        return launch_gram_x3(Sx, Sy, n_b, p, q, sc.mx, sc.my, sc.dx, sc.dy, coef, fresh, M_xx, M_xy, bd, s);
    }
    for (int phase = 0; phase < 2; ++phase) {
        const float* shx = phase ? sc.cx : nullptr;
        const float* shy = phase ? sc.cy : nullptr;
        hipLaunchKernelGGL(colsum_kernel<false>, gx, dim3(CS_THREADS), 0, s, X, n_b, p, shx, sc.part, stride, 0,
                           nullptr);
        hipLaunchKernelGGL(colsum_kernel<false>, gy, dim3(CS_THREADS), 0, s, Y, n_b, q, shy, sc.part, stride, p,
                           (phase == 1 && ss_y) ? sc.part2 : nullptr);
        hipLaunchKernelGGL(colsum_finalize_kernel, dim3(fin), dim3(256), 0, s, sc.part, sc.splits, p, q,
                           n_b, n_old, phase, 0, sc.cx, sc.cy, sc.mx, sc.my, sc.dx, sc.dy, mean_x, mean_y,
                           sc.part2, phase == 1 ? ss_y : nullptr);
    }
    const int nTx = (p + GT - 1) / GT, nTy = (q + GT - 1) / GT;
    const int nTb = bd ? (bd + GT - 1) / GT : 0;
    const int nXX = bd ? (p / bd) * (nTb * (nTb + 1) / 2) : nTx * (nTx + 1) / 2;
    const int blocks = nXX + nTx * nTy;
    hipLaunchKernelGGL(gram_kernel<false>, dim3(blocks), dim3(256), 0, s, X, Y, n_b, p, q, sc.cx, sc.cy,
                       sc.mx, sc.my, sc.dx, sc.dy, coef, fresh, M_xx, M_xy, nTx, nXX, bd, nTb);
    return hipGetLastError();
}

// ---- merging two states ----------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_delta_kernel(int p, int q, double frac, int fresh,
                                                          float* __restrict__ mean_x,
                                                          float* __restrict__ mean_y,
                                                          const float* __restrict__ s_mean_x,
                                                          const float* __restrict__ s_mean_y,
                                                          float* __restrict__ dx,
                                                          float* __restrict__ dy, float* __restrict__ ss_y,
                                                          const float* __restrict__ s_ss_y, double coef) {
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= p + q) return;
    const bool isx = col < p;
    const int c = isx ? col : col - p;
    float* mean = isx ? mean_x : mean_y;
    const float* sm = isx ? s_mean_x : s_mean_y;
    float* d = isx ? dx : dy;
    if (fresh) {
        d[c] = 0.f;
        mean[c] = sm[c];
        if (!isx && ss_y) ss_y[c] = s_ss_y[c];
        return;
    }
    const double delta = (double)sm[c] - (double)mean[c];
    d[c] = (float)delta;
    mean[c] = (float)((double)mean[c] + delta * frac);
    if (!isx && ss_y) ss_y[c] = (float)((double)ss_y[c] + (double)s_ss_y[c] + coef * delta * delta);
}

__global__ __launch_bounds__(256) void merge_moments_kernel(int rows, int cols, float coef,
                                                            int fresh, float* __restrict__ M,
                                                            const float* __restrict__ S,
                                                            const float* __restrict__ da,
                                                            const float* __restrict__ db) {
    const int64_t n = (int64_t)rows * cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += stride) {
        const int i = (int)(idx / cols), j = (int)(idx - (int64_t)i * cols);
        const float v = S[idx] + coef * da[i] * db[j];
        M[idx] = fresh ? S[idx] : M[idx] + v;
    }
}

hipError_t launch_gram_merge(int p, int q, int64_t n_dst, int64_t n_src, float* mean_x,
                             float* mean_y, float* M_xx, float* M_xy, float* ss_y, const float* s_mean_x,
                             const float* s_mean_y, const float* s_M_xx, const float* s_M_xy, const float* s_ss_y,
                             int bd, const GramScratch& sc, hipStream_t s) {
    const double n = (double)n_dst + (double)n_src;
    const int fresh = (n_dst == 0);
    const float coef = (float)((double)n_dst * (double)n_src / n);
    hipLaunchKernelGGL(merge_delta_kernel, dim3((p + q + 255) / 256), dim3(256), 0, s, p, q,
                       (double)n_src / n, fresh, mean_x, mean_y, s_mean_x, s_mean_y, sc.dx, sc.dy, ss_y, s_ss_y,
                       (double)n_dst * (double)n_src / n);
    if (bd) {
        for (int b = 0; b < p / bd; ++b)
            hipLaunchKernelGGL(merge_moments_kernel, dim3(1024), dim3(256), 0, s, bd, bd, coef, fresh,
                               M_xx + (size_t)b * bd * bd, s_M_xx + (size_t)b * bd * bd, sc.dx + (size_t)b * bd,
                               sc.dx + (size_t)b * bd);
    } else {
        hipLaunchKernelGGL(merge_moments_kernel, dim3(4096), dim3(256), 0, s, p, p, coef, fresh, M_xx, s_M_xx,
                           sc.dx, sc.dx);
    }
    hipLaunchKernelGGL(merge_moments_kernel, dim3(4096), dim3(256), 0, s, p, q, coef, fresh, M_xy, s_M_xy,
                       sc.dx, sc.dy);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace kvmap
