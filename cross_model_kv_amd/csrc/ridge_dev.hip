// Ridge solve on the device, in float64 (KVBridge README, fitting section: one closed-form
// ridge per target, W = (M_xx + lambda I)^-1 M_xy with an unpenalised intercept
// b = mean_y - mean_x W).
//
//   A = sym(M_xx) + lambda I  (read from M_xx's upper triangle, like the host solver), padded to a
//       multiple of 64 with an identity block;  B = M_xy, padded with zero rows/columns
//   A = L L^T    right-looking blocked Cholesky, 64-wide blocks: factor the diagonal block in
//                one workgroup, solve the panel below it, update the trailing lower triangle
//   L Z = B, L^T W = Z   blocked forward / back substitution over all right-hand sides
//   b = mean_y - mean_x W;  W written output-major [q][p] in bf16 or fp32 (the apply's layout),
//   or, for layer scoring, the in-sample R^2 of the fit pooled over groups of y columns, from
//   the statistics alone: RSS_c = ss_y[c] - w_c . M_xy[:, c] - lambda |w_c|^2
// Every update is a 64 x 64 fp64 tile C -= op(A) op(B) with K = 64 on the vector ALUs
// (fp64 FMA runs at the same rate as the fp64 matrix cores on this chip).  A non-positive or
// non-finite pivot sets a device flag that the host turns into KVMAP_ERR_NOT_SPD.

#include "common.h"
#include "internal.h"

namespace kvmap {

namespace {

constexpr int RB = 64;  // block size

// Upper-triangle index of the lower-triangle tile list: tile u -> (I >= J)
__device__ __forceinline__ void lower_decode(int u, int& I, int& J) {
    int i = (int)((sqrt(8.0 * (double)u + 1.0) - 1.0) * 0.5);
    while ((int64_t)i * (i + 1) / 2 > u) --i;
    while ((int64_t)(i + 1) * (i + 2) / 2 <= u) ++i;
    I = i;
    J = u - (int)((int64_t)i * (i + 1) / 2);
}

}  // namespace

// A[i][j] = M_xx[min][max] (+ lambda on the diagonal) for i, j < p; identity padding.
__global__ __launch_bounds__(256) void ridge_init_a_kernel(const float* __restrict__ M_xx, int p, int P,
                                                           double lambda, double* __restrict__ A) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)P * P) return;
    const int i = (int)(idx / P), j = (int)(idx - (int64_t)i * P);
    double v;
    if (i < p && j < p) {
        v = (double)M_xx[(size_t)min(i, j) * p + max(i, j)];
        if (i == j) v += lambda;
    } else {
        v = (i == j) ? 1.0 : 0.0;
    }
    A[idx] = v;
}

__global__ __launch_bounds__(256) void ridge_init_b_kernel(const float* __restrict__ M_xy, int p, int q, int P,
                                                           int Q, double* __restrict__ B) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)P * Q) return;
    const int i = (int)(idx / Q), c = (int)(idx - (int64_t)i * Q);
    B[idx] = (i < p && c < q) ? (double)M_xy[(size_t)i * q + c] : 0.0;
}

// Factor the diagonal block kb in place (lower triangle), one workgroup of 64 threads.
__global__ __launch_bounds__(64) void ridge_potrf_kernel(double* __restrict__ A, int P, int kb,
                                                         int* __restrict__ bad) {
    __shared__ double t[RB][RB + 1];
    const int r = threadIdx.x;
    const int o = kb * RB;
    for (int c = 0; c < RB; ++c) t[r][c] = A[(size_t)(o + r) * P + o + c];
    __syncthreads();
    for (int j = 0; j < RB; ++j) {
        double d = t[j][j];
        if (!(d > 0.0) || !isfinite(d)) {
            if (r == 0) atomicOr(bad, 1);
            d = 1.0;  // keep going with a harmless pivot; the result is refused by the host
        }
        const double ljj = sqrt(d);
        __syncthreads();
        if (r == j) t[j][j] = ljj;
        if (r > j) t[r][j] /= ljj;
        __syncthreads();
        if (r > j)
            for (int m = j + 1; m <= r; ++m) t[r][m] -= t[r][j] * t[m][j];
        __syncthreads();
    }
    for (int c = 0; c < RB; ++c) A[(size_t)(o + r) * P + o + c] = (c <= r) ? t[r][c] : 0.0;
}

// Panel: A_ik <- A_ik L_kk^-T for the 64-row blocks i below kb; workgroup = one row block,
// thread = one row (forward substitution along the row).
__global__ __launch_bounds__(64) void ridge_trsm_panel_kernel(double* __restrict__ A, int P, int kb) {
    __shared__ double L[RB][RB + 1];
    __shared__ double X[RB][RB + 1];
    const int r = threadIdx.x;
    const int o = kb * RB;
    const int i0 = o + RB * (1 + (int)blockIdx.x);
    for (int c = 0; c < RB; ++c) {
        L[r][c] = A[(size_t)(o + r) * P + o + c];
        X[r][c] = A[(size_t)(i0 + r) * P + o + c];
    }
    __syncthreads();
    for (int j = 0; j < RB; ++j) {
        double s = X[r][j];
        for (int m = 0; m < j; ++m) s -= X[r][m] * L[j][m];
        X[r][j] = s / L[j][j];
    }
    for (int c = 0; c < RB; ++c) A[(size_t)(i0 + r) * P + o + c] = X[r][c];
}

// Right-hand sides, diagonal block kb: forward (Z_kb = L_kk^-1 B_kb) or backward
// (W_kb = L_kk^-T Z_kb); workgroup = 64 right-hand-side columns, thread = one column.
template <bool FWD>
__global__ __launch_bounds__(64) void ridge_trsm_rhs_kernel(const double* __restrict__ A, int P,
                                                            double* __restrict__ B, int Q, int kb) {
    __shared__ double L[RB][RB + 1];
    __shared__ double Xs[RB][RB + 1];
    const int c = threadIdx.x;
    const int o = kb * RB, c0 = (int)blockIdx.x * RB;
    for (int rr = 0; rr < RB; ++rr) {
        L[rr][c] = A[(size_t)(o + rr) * P + o + c];
        Xs[rr][c] = B[(size_t)(o + rr) * Q + c0 + c];
    }
    __syncthreads();
    if (FWD) {
        for (int rr = 0; rr < RB; ++rr) {
            double s = Xs[rr][c];
            for (int m = 0; m < rr; ++m) s -= L[rr][m] * Xs[m][c];
            Xs[rr][c] = s / L[rr][rr];
        }
    } else {
        for (int rr = RB - 1; rr >= 0; --rr) {
            double s = Xs[rr][c];
            for (int m = rr + 1; m < RB; ++m) s -= L[m][rr] * Xs[m][c];
            Xs[rr][c] = s / L[rr][rr];
        }
    }
    for (int rr = 0; rr < RB; ++rr) B[(size_t)(o + rr) * Q + c0 + c] = Xs[rr][c];
}

// C -= op(A) op(B) on 64 x 64 tiles, K = 64.  op(A)[r][m] = Aop[r * sar + m * sam],
// op(B)[m][c] = Bop[m * sbm + c * sbc] (one stride of each is 1).  The tile list:
//   MODE 0  trailing lower triangle of A after block kb:  C = A_IJ, op(A) = A_I,kb,
//           op(B) = A_J,kb^T  (I >= J > kb)
//   MODE 1  forward update of the right-hand sides: C = B_I,J (I > kb), op(A) = L_I,kb,
//           op(B) = Z_kb,J
//   MODE 2  backward update: C = Z_I,J (I < kb), op(A) = L_kb,I^T, op(B) = W_kb,J
// 256 threads; thread (ty, tx) accumulates rows 4 ty .. 4 ty + 3, columns 4 tx .. 4 tx + 3.
template <int MODE>
__global__ __launch_bounds__(256) void ridge_update_kernel(double* __restrict__ A, int P, double* __restrict__ B,
                                                           int Q, int kb, int ncol) {
    __shared__ double As[RB][RB + 4];  // [m][r]
    __shared__ double Bs[RB][RB + 4];  // [m][c]
    const int tid = threadIdx.x;
    int I, J;
    if (MODE == 0) {
        lower_decode(blockIdx.x, I, J);
        I += kb + 1;
        J += kb + 1;
    } else {
        I = (int)blockIdx.x / ncol;
        J = (int)blockIdx.x - I * ncol;
        if (MODE == 1) I += kb + 1;
    }
    const int o = kb * RB;
    double* C;
    int ldc;
    const double* Ap;
    int sar, sam;
    const double* Bp;
    int sbm, sbc;
    if (MODE == 0) {
        C = A + (size_t)I * RB * P + (size_t)J * RB;
        ldc = P;
        Ap = A + (size_t)I * RB * P + o; sar = P; sam = 1;
        Bp = A + (size_t)J * RB * P + o; sbm = 1; sbc = P;
    } else if (MODE == 1) {
        C = B + (size_t)I * RB * Q + (size_t)J * RB;
        ldc = Q;
        Ap = A + (size_t)I * RB * P + o; sar = P; sam = 1;
        Bp = B + (size_t)o * Q + (size_t)J * RB; sbm = Q; sbc = 1;
    } else {
        C = B + (size_t)I * RB * Q + (size_t)J * RB;
        ldc = Q;
        Ap = A + (size_t)o * P + (size_t)I * RB; sar = 1; sam = P;
        Bp = B + (size_t)o * Q + (size_t)J * RB; sbm = Q; sbc = 1;
    }
    // loads: 4096 elements each, 16 per thread, consecutive threads along the unit stride
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int e = u * 256 + tid;
        const int x = e >> 6, y = e & 63;  // y runs along the unit stride
        if (sam == 1) As[y][x] = Ap[(size_t)x * sar + y];  // element (r = x, m = y)
        else As[x][y] = Ap[(size_t)x * sam + y];           // element (m = x, r = y)
        if (sbc == 1) Bs[x][y] = Bp[(size_t)x * sbm + y];  // element (m = x, c = y)
        else Bs[y][x] = Bp[(size_t)x * sbc + y];           // element (c = x, m = y)
    }
    __syncthreads();
    const int ty = tid >> 4, tx = tid & 15;
    double acc[4][4] = {};
#pragma unroll 8
    for (int m = 0; m < RB; ++m) {
        double a[4], b[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            a[v] = As[m][ty * 4 + v];
            b[v] = Bs[m][tx * 4 + v];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) acc[r][cc] = fma(a[r], b[cc], acc[r][cc]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) C[(size_t)(ty * 4 + r) * ldc + tx * 4 + cc] -= acc[r][cc];
}

// b[c] = mean_y[c] - sum_i mean_x[i] W[i][c] (fp64), and W_out[c][i] = W[i][c] in the output
// dtype (output-major), through a 64 x 64 transpose in LDS.  Workgroup: 64 columns c x all i.
template <bool BF16>
__global__ __launch_bounds__(256) void ridge_finalize_kernel(const double* __restrict__ W, int P, int Q, int p,
                                                             int q, const float* __restrict__ mean_x,
                                                             const float* __restrict__ mean_y,
                                                             void* __restrict__ W_out, void* __restrict__ b_out) {
    __shared__ double t[RB][RB + 1];
    __shared__ double part[4][RB];
    const int tid = threadIdx.x;
    const int c0 = (int)blockIdx.x * RB;
    const int cx = tid & 63, ry = tid >> 6;  // 4 row groups
    double dot = 0.0;
    for (int i0 = 0; i0 < p; i0 += RB) {
        for (int rr = ry; rr < RB; rr += 4) {
            const int i = i0 + rr;
            const double w = (i < p) ? W[(size_t)i * Q + c0 + cx] : 0.0;
            t[rr][cx] = w;
            if (i < p) dot += (double)mean_x[i] * w;
        }
        __syncthreads();
        // write rows c of W_out: thread (ry, cx) writes element i0 + cx of columns c0 + ry + 4k
        for (int cc = ry; cc < RB; cc += 4) {
            const int c = c0 + cc, i = i0 + cx;
            if (c < q && i < p) {
                const double v = t[cx][cc];
                if (BF16) ((uint16_t*)W_out)[(size_t)c * p + i] = (uint16_t)(pack_bf16((float)v, 0.f) & 0xffffu);
                else ((float*)W_out)[(size_t)c * p + i] = (float)v;
            }
        }
        __syncthreads();
    }
    part[ry][cx] = dot;
    __syncthreads();
    if (ry == 0 && c0 + cx < q) {
        const double bv = (double)mean_y[c0 + cx] - (part[0][cx] + part[1][cx] + part[2][cx] + part[3][cx]);
        if (BF16) ((uint16_t*)b_out)[c0 + cx] = (uint16_t)(pack_bf16((float)bv, 0.f) & 0xffffu);
        else ((float*)b_out)[c0 + cx] = (float)bv;
    }
}

// In-sample residual sum of squares of column c from the statistics alone.  With
// yc = y - mean_y, xc = x - mean_x and (M_xx + lambda I) w = m (m = M_xy[:, c]):
//   sum (yc - xc w)^2 = ss_y[c] - 2 w.m + w^T M_xx w = ss_y[c] - w.m - lambda |w|^2,
// since w^T M_xx w = w^T (m - lambda w).  Workgroup: 64 columns; the 4 row groups are
// reduced in a fixed order.
__global__ __launch_bounds__(256) void ridge_rss_kernel(const double* __restrict__ W, int Q, int p, int q,
                                                        const float* __restrict__ M_xy,
                                                        const float* __restrict__ ss_y, double lambda,
                                                        double* __restrict__ rss) {
    __shared__ double pd[4][RB];
    __shared__ double pn[4][RB];
    const int tid = threadIdx.x;
    const int cx = tid & 63, ry = tid >> 6;
    const int c = (int)blockIdx.x * RB + cx;
    double dot = 0.0, nrm = 0.0;
    if (c < q) {
        for (int i = ry; i < p; i += 4) {
            const double w = W[(size_t)i * Q + c];
            dot += w * (double)M_xy[(size_t)i * q + c];
            nrm += w * w;
        }
    }
    pd[ry][cx] = dot;
    pn[ry][cx] = nrm;
    __syncthreads();
    if (ry == 0 && c < q) {
        const double d = ((pd[0][cx] + pd[1][cx]) + pd[2][cx]) + pd[3][cx];
        const double n2 = ((pn[0][cx] + pn[1][cx]) + pn[2][cx]) + pn[3][cx];
        rss[c] = (double)ss_y[c] - d - lambda * n2;
    }
}

// R^2 of group g (columns g*group .. g*group + group - 1) pooled over its columns:
// 1 - sum RSS / sum ss_y; NaN when the group's total sum of squares is 0.
__global__ __launch_bounds__(256) void ridge_r2_group_kernel(const double* __restrict__ rss,
                                                             const float* __restrict__ ss_y, int groups,
                                                             int group, double* __restrict__ r2) {
    const int g = (int)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    double r = 0.0, t = 0.0;
    for (int j = 0; j < group; ++j) {
        r += rss[(size_t)g * group + j];
        t += (double)ss_y[(size_t)g * group + j];
    }
    r2[g] = t > 0.0 ? 1.0 - r / t : __builtin_nan("");
}

// ---------------------------------------------------------------------------------------

size_t ridge_dev_scratch_bytes(int p, int q) {
    const size_t P = ((size_t)p + RB - 1) / RB * RB, Q = ((size_t)q + RB - 1) / RB * RB;
    return (P * P + P * Q + Q) * sizeof(double) + 256;  // A, B (then W), rss, pivot flag
}

// A = sym(M_xx) + lambda I = L L^T (lower triangle of A), then W = A^-1 M_xy in B = A + P^2,
// row-major [P][Q].
static void ridge_dev_solve(int p, int q, const float* M_xx, const float* M_xy, double lambda, void* scratch,
                            int* bad, hipStream_t s) {
    const int P = (p + RB - 1) / RB * RB, Q = (q + RB - 1) / RB * RB;
    const int nb = P / RB, nq = Q / RB;
    double* A = (double*)scratch;
    double* B = A + (size_t)P * P;
    hipLaunchKernelGGL(ridge_init_a_kernel, dim3((unsigned)(((int64_t)P * P + 255) / 256)), dim3(256), 0, s, M_xx, p,
                       P, lambda, A);
    hipLaunchKernelGGL(ridge_init_b_kernel, dim3((unsigned)(((int64_t)P * Q + 255) / 256)), dim3(256), 0, s, M_xy, p,
                       q, P, Q, B);
    for (int kb = 0; kb < nb; ++kb) {
        hipLaunchKernelGGL(ridge_potrf_kernel, dim3(1), dim3(RB), 0, s, A, P, kb, bad);
        const int below = nb - kb - 1;
        if (below > 0) {
            hipLaunchKernelGGL(ridge_trsm_panel_kernel, dim3(below), dim3(RB), 0, s, A, P, kb);
            hipLaunchKernelGGL(ridge_update_kernel<0>, dim3(below * (below + 1) / 2), dim3(256), 0, s, A, P, B, Q,
                               kb, 0);
        }
    }
    for (int kb = 0; kb < nb; ++kb) {
        hipLaunchKernelGGL(ridge_trsm_rhs_kernel<true>, dim3(nq), dim3(RB), 0, s, A, P, B, Q, kb);
        const int below = nb - kb - 1;
        if (below > 0)
            hipLaunchKernelGGL(ridge_update_kernel<1>, dim3(below * nq), dim3(256), 0, s, A, P, B, Q, kb, nq);
    }
    for (int kb = nb - 1; kb >= 0; --kb) {
        hipLaunchKernelGGL(ridge_trsm_rhs_kernel<false>, dim3(nq), dim3(RB), 0, s, A, P, B, Q, kb);
        if (kb > 0) hipLaunchKernelGGL(ridge_update_kernel<2>, dim3(kb * nq), dim3(256), 0, s, A, P, B, Q, kb, nq);
    }
}

hipError_t launch_ridge_dev(int p, int q, const float* mean_x, const float* mean_y, const float* M_xx,
                            const float* M_xy, double lambda, void* W_out, void* b_out, bool bf16,
                            void* scratch, int* bad, hipStream_t s) {
    const int P = (p + RB - 1) / RB * RB, Q = (q + RB - 1) / RB * RB;
    const int nq = Q / RB;
    const double* B = (const double*)scratch + (size_t)P * P;
    ridge_dev_solve(p, q, M_xx, M_xy, lambda, scratch, bad, s);
    if (bf16)
        hipLaunchKernelGGL(ridge_finalize_kernel<true>, dim3(nq), dim3(256), 0, s, B, P, Q, p, q, mean_x, mean_y,
                           W_out, b_out);
    else
        hipLaunchKernelGGL(ridge_finalize_kernel<false>, dim3(nq), dim3(256), 0, s, B, P, Q, p, q, mean_x, mean_y,
                           W_out, b_out);
    return hipGetLastError();
}

hipError_t launch_ridge_r2(int p, int q, const float* M_xx, const float* M_xy, const float* ss_y, double lambda,
                           int group, double* r2_out, void* scratch, int* bad, hipStream_t s) {
    const int P = (p + RB - 1) / RB * RB, Q = (q + RB - 1) / RB * RB;
    const double* B = (const double*)scratch + (size_t)P * P;
    double* rss = (double*)scratch + (size_t)P * P + (size_t)P * Q;
    ridge_dev_solve(p, q, M_xx, M_xy, lambda, scratch, bad, s);
    hipLaunchKernelGGL(ridge_rss_kernel, dim3(Q / RB), dim3(256), 0, s, B, Q, p, q, M_xy, ss_y, lambda, rss);
    const int groups = q / group;
    hipLaunchKernelGGL(ridge_r2_group_kernel, dim3((groups + 255) / 256), dim3(256), 0, s, rss, ss_y, groups, group,
                       r2_out);
    return hipGetLastError();
}

}  // namespace kvmap
