// Ridge solve on the device, in float64 (KVBridge README, fitting section: one closed-form
// ridge per target, W = (M_xx + lambda I)^-1 M_xy with an unpenalised intercept
// b = mean_y - mean_x W).
//
//   A = sym(M_xx) + lambda I  (read from M_xx's upper triangle, like the host solver), padded to a
//       multiple of 128 with an identity block;  B = M_xy, padded with zero rows/columns
//   A = L L^T    right-looking blocked Cholesky, 64-wide blocks: factor the diagonal block and
//                invert its factor in one workgroup, multiply the panel below it by that
//                inverse, update the trailing lower triangle (once per panel of 4 blocks)
//   L Z = B, L^T W = Z   blocked forward / back substitution over all right-hand sides, each
//                diagonal step a product with the block's inverse
//   b = mean_y - mean_x W;  W written output-major [q][p] in bf16 or fp32 (the apply's layout),
//   or, for layer scoring, the in-sample R^2 of the fit pooled over groups of y columns, from
//   the statistics alone: RSS_c = ss_y[c] - w_c . M_xy[:, c] - lambda |w_c|^2
// A batch of up to kRidgeMaxBatch systems of one shape runs through every kernel together
// (the last grid dimension = system): the 64-wide diagonal steps form a serial chain of about
// 4 P / 64 small launches, which a batch pays once.  The tile updates C -= op(A) op(B) run on the
// fp64 matrix cores (v_mfma_f64_16x16x4f64), operands staged through LDS in their global
// orientation: 64 x 64 tiles inside a panel, 128 x 128 tiles for the once-per-panel updates of
// the trailing matrix and of the right-hand sides.  A non-positive or
// non-finite pivot sets the system's device flag, which the host turns into KVMAP_ERR_NOT_SPD.

#include <algorithm>
#include <utility>
#include <vector>

#include "common.h"
#include "internal.h"

namespace kvmap {

namespace {

constexpr int RB = 64;       // block size
// LDS row strides (doubles) of staged tiles, odd: a 16-lane group of a fragment read (one
// double per lane, lanes 16 rows apart by one row each) then covers 16 distinct bank pairs of
// the 32 banks; with an even stride of 66, rows 8 apart shared a pair (the counters showed 40 %
// of the LDS cycles of the trailing update in bank conflicts)
constexpr int LDW = RB + 1;  // 64 x 64 tile
constexpr int TB = 128;      // C tile of the large updates (the trailing matrix, the right-hand sides)
constexpr int LD_M = TB + 2;  // LDS row stride of a large-update stage stored with its K index as rows

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// Everything a batched launch needs, passed by value (kernel argument space).
struct RidgeArgs {
    RidgeSys s[kRidgeMaxBatch];
    double* scratch;  // system z: A = scratch + z * stride, B = A + P^2, rss = B + P Q, Li = rss + Q
    size_t stride;    // doubles per system
    int* bad;         // [n] pivot flags
    int p, q, P, Q;
    double lambda;
};

// Every kernel of the solve takes its system from grid y: these helpers index the scratch by blockIdx.y.
__device__ __forceinline__ double* sys_a(const RidgeArgs& g) { return g.scratch + (size_t)blockIdx.y * g.stride; }
__device__ __forceinline__ double* sys_b(const RidgeArgs& g) { return sys_a(g) + (size_t)g.P * g.P; }
__device__ __forceinline__ double* sys_rss(const RidgeArgs& g) {
    return sys_b(g) + (size_t)g.P * g.Q;
}
// Inverses of the 64 x 64 diagonal blocks of L, [P / 64][64][64]
__device__ __forceinline__ double* sys_li(const RidgeArgs& g) { return sys_rss(g) + g.Q; }

// Lower-triangle tile list after a block: tile u -> (I >= J)
__device__ __forceinline__ void lower_decode(int u, int& I, int& J) {
    int i = (int)((sqrt(8.0 * (double)u + 1.0) - 1.0) * 0.5);
    while ((int64_t)i * (i + 1) / 2 > u) --i;
    while ((int64_t)(i + 1) * (i + 2) / 2 <= u) ++i;
    I = i;
    J = u - (int)((int64_t)i * (i + 1) / 2);
}

}  // namespace

// A[i][j] = M_xx[min][max] (+ lambda on the diagonal) for i, j < p; identity padding.  Only the
// 64 x 64 tiles on and below the diagonal are written: no kernel of the solve reads A above its
// diagonal blocks (the large trailing update computes its diagonal 128 x 128 tiles whole, and
// their upper 64 x 64 quarter is never read).  One tile (I, J), I >= J, per workgroup: the tile
// is read from M_xx's upper triangle as tile (J, I) -- rows of 64 consecutive floats -- through
// LDS, so that the transposed tile is read and written with whole rows too.
__global__ __launch_bounds__(256) void ridge_init_a_kernel(const RidgeArgs g) {
    __shared__ float t[RB][RB + 1];
    const int P = g.P, p = g.p;
    int I, J;
    lower_decode((int)blockIdx.x, I, J);
    const float* M_xx = g.s[blockIdx.y].M_xx;
    const int tr = min(I, J) * RB, tc = max(I, J) * RB;  // source tile in the upper triangle
    const int tid = threadIdx.x, c = tid & 63;
    for (int r = tid >> 6; r < RB; r += 4) {
        const int i = tr + r, j = tc + c;
        t[r][c] = (i < p && j < p) ? M_xx[(size_t)i * p + j] : 0.f;
    }
    __syncthreads();
    double* A = sys_a(g);
    for (int r = tid >> 6; r < RB; r += 4) {
        const int i = I * RB + r, j = J * RB + c;
        double v;
        if (i < p && j < p) {
            // element (i, j) = M_xx[min][max]: in the staged tile at (i - tr, j - tc) when i <= j
            // (the tile is (I, J) itself, or the diagonal tile's upper part), else at (j - tr, i - tc)
            v = (i <= j) ? (double)t[i - tr][j - tc] : (double)t[j - tr][i - tc];
            if (i == j) v += g.lambda;
        } else {
            v = (i == j) ? 1.0 : 0.0;
        }
        A[(size_t)i * P + j] = v;
    }
}

__global__ __launch_bounds__(256) void ridge_init_b_kernel(const RidgeArgs g) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int P = g.P, Q = g.Q, p = g.p, q = g.q;
    if (idx >= (int64_t)P * Q) return;
    const float* M_xy = g.s[blockIdx.y].M_xy;
    const int i = (int)(idx / Q), c = (int)(idx - (int64_t)i * Q);
    sys_b(g)[idx] = (i < p && c < q) ? (double)M_xy[(size_t)i * q + c] : 0.0;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1 / sqrt(d) for d > 0 in float64: the hardware estimate refined by two Newton steps
// y <- y (3 - d y^2) / 2, each of which doubles the correct bits of the estimate.
__device__ __forceinline__ double rsqrt_f64(double d) {
    double y = __builtin_amdgcn_rsq(d);
    y = y * fma(-0.5 * d * y, y, 1.5);
    y = y * fma(-0.5 * d * y, y, 1.5);
    return y;
}

// Factor the diagonal block kb in place (lower triangle) and write the inverse of the factor to
// Li[kb]; one workgroup of 4 waves per system.  The inverse turns every triangular solve with
// this block (the panel below it and both substitutions) into a 64 x 64 tile product on the
// matrix cores.  The block sits in LDS (odd row stride) and is factored in 16-wide sub-blocks
// (right-looking), so that the bulk of the work is 16 x 16 x 16 products on the fp64 matrix
// cores and only 16-step chains stay serial.  For each diagonal sub-block k:
//   wave 0 factors it, 16 lanes holding its rows in registers: step j publishes column j as it
//     stands (a_mj, m > j) to col[], reads the pivot a_jj from lane j with v_readlane, takes
//     rj = 1 / sqrt(a_jj), l_rj = a_rj rj (l_jj = a_jj rj = sqrt(a_jj), one reciprocal square
//     root doing for the root and the division), and every row lane r updates
//     a_rm -= (l_rj rj) a_mj for m > j.  The next pivot comes from lane j + 1's own registers,
//     so the chain of pivots never waits for the LDS round trip;
//   in the same steps, on 16 more lanes, it inverts the factor by right-looking substitution,
//     lane r holding column r of the inverse: x_j = v_j rj, then v_m -= (x_j rj) a_mj for m > j
//     (= l_mj x_j), starting from v = e_r;
//   the sub-blocks below, as transposes: L_ik^T = X_kk A_ik^T (X = L^-1), one per wave;
//   the trailing sub-blocks: A_ij -= L_ik L_jk^T (k < j <= i).  Wave 0 updates the next
//     diagonal sub-block from its own panel in registers and factors it at once, while waves
//     1-3 update the other trailing sub-blocks and the inverse's sub-blocks of row k,
//     X_km = -X_kk (sum over n = m .. k-1 of L_kn X_nm) for m < k.
// Two barriers per sub-block: after the factor (and the other waves' work beside it), and after
// the panels.  Within a wave, LDS operations complete in issue order; a compiler memory fence
// keeps the compiler from moving them across phases.
// v_mfma_f64_16x16x4f64: lane (i, k) = (lane & 15, lane >> 4) supplies A[i][k] and B[k][i] of
// each K = 4 step; accumulator element e of the lane is D[(lane >> 4) + 4 e][lane & 15].  Element
// e of a product D is then what the lane supplies at step e of the next product for B = D or for
// A = D^T, so products chain in registers.  Elements above the diagonal of a diagonal sub-block
// are updated too and never used.
__global__ __launch_bounds__(256) void ridge_potrf_kernel(const RidgeArgs g, int kb) {
    constexpr int SB = 16;         // sub-block
    static_assert(RB / SB == 4, "the phases below are written out for 4 sub-blocks per side");
    constexpr int LDL = RB + 1;    // LDS row stride (doubles)
    __shared__ double Ls[RB * LDL];  // the block: A in, L out (lower triangle)
    __shared__ double Xs[RB * LDL];  // X = L^-1 (lower triangle; the rest is not written)
    __shared__ double col[64];       // col[m], m < 16: the published column (lanes 16.. write copies)
    double* A = sys_a(g);
    const int P = g.P;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const bool isrow = (lane & 16) == 0;
    const int o = kb * RB;
    auto fence = []() { asm volatile("" ::: "memory"); };
    const f64x4_t zero4 = {0.0, 0.0, 0.0, 0.0};
    {   // rows 16 w .. 16 w + 15 of the block (coalesced rows)
        double v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = A[(size_t)(o + 16 * w + i) * P + o + lane];
#pragma unroll
        for (int i = 0; i < 16; ++i) Ls[(16 * w + i) * LDL + lane] = v[i];
    }
    fence();
    // wave 0: factor diagonal sub-block k and invert its factor (Ls rows, Xs columns)
    auto factor = [&](const int k) {
        const int k0 = k * SB;
        // lanes with bit 4 clear hold row r (y = a_r.), the others column r of the inverse
        // (y = v_.r); lanes 32.. repeat lanes 0..31.  One instruction updates both.
        double y[SB];
#pragma unroll
        for (int c = 0; c < SB; ++c) {
            double a = Ls[(k0 + r) * LDL + k0 + c];
            asm volatile("" : "+v"(a));  // load on every lane (no branch), then select
            y[c] = isrow ? a : (c == r ? 1.0 : 0.0);
        }
        fence();
        double piv = readlane_f64(y[0], 0);
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            // column j as it stands (a_mj, m > j), for every lane; its LDS round trip runs
            // while the pivot's reciprocal square root is computed
            const double aj = y[j];
            col[lane] = aj;
            fence();
            double cm[SB];
#pragma unroll
            for (int m = j + 1; m < SB; ++m) cm[m] = col[m];
            __builtin_amdgcn_sched_barrier(0);
            // rows: l_rj = a_rj rj, and lane j's own a_jj is the pivot, so l_jj = a_jj rj =
            // sqrt(a_jj); inverse columns: x_j = v_j rj.  The multiplier s = y_j rj makes
            // a_rm -= s a_mj the update -= l_rj l_mj and v_m -= s a_mj the update -= l_mj x_j.
            const double rj = rsqrt_f64(piv);
            y[j] = aj * rj;
            const double sc = y[j] * rj;
            // The next pivot is lane j + 1's a_(j+1)(j+1) - s a_(j+1)j, whose column value is its
            // own aj: the same operands as its update from col below, so the same result (the
            // lane's own a_(j+1)(j+1) in the next step), with no wait for the LDS round trip.
            if (j + 1 < SB) piv = readlane_f64(fma(-sc, aj, y[j + 1]), j + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = j + 1; m < SB; ++m) y[m] = fma(-sc, cm[m], y[m]);
            fence();
        }
        // rows of the factor (zero above the diagonal) to Ls, columns of the inverse to Xs;
        // lanes 32.. store the same values to the same places
#pragma unroll
        for (int c = 0; c < SB; ++c) {
            double* dst = isrow ? &Ls[(k0 + r) * LDL + k0 + c] : &Xs[(k0 + c) * LDL + k0 + r];
            *dst = (isrow && c > r) ? 0.0 : y[c];
        }
        fence();
    };
    // D = L_ik^T = X_kk A_ik^T, and L_ik stored over A_ik
    auto panel = [&](const int k, const int i) {
        const int k0 = k * SB;
        f64x4_t D = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            D = __builtin_amdgcn_mfma_f64_16x16x4f64(Xs[(k0 + r) * LDL + k0 + 4 * s + kq],
                                                     Ls[(i * SB + r) * LDL + k0 + 4 * s + kq], D, 0, 0, 0);
        fence();
#pragma unroll
        for (int e = 0; e < 4; ++e) Ls[(i * SB + r) * LDL + k0 + kq + 4 * e] = D[e];
        fence();
        return D;
    };
    // A_ij -= L_ik L_jk^T, the operands from Ls
    auto trail = [&](const int k, const int i, const int j) {
        const int k0 = k * SB;
        f64x4_t C;
#pragma unroll
        for (int e = 0; e < 4; ++e) C[e] = Ls[(i * SB + kq + 4 * e) * LDL + j * SB + r];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            C = __builtin_amdgcn_mfma_f64_16x16x4f64(-Ls[(i * SB + r) * LDL + k0 + 4 * s + kq],
                                                     Ls[(j * SB + r) * LDL + k0 + 4 * s + kq], C, 0, 0, 0);
        fence();
#pragma unroll
        for (int e = 0; e < 4; ++e) Ls[(i * SB + kq + 4 * e) * LDL + j * SB + r] = C[e];
        fence();
    };
    // A_ii -= L_ik L_ik^T with D = L_ik^T in registers
    auto trail_diag = [&](const int i, const f64x4_t D) {
        f64x4_t C;
#pragma unroll
        for (int e = 0; e < 4; ++e) C[e] = Ls[(i * SB + kq + 4 * e) * LDL + i * SB + r];
#pragma unroll
        for (int s = 0; s < 4; ++s) C = __builtin_amdgcn_mfma_f64_16x16x4f64(-D[s], D[s], C, 0, 0, 0);
        fence();
#pragma unroll
        for (int e = 0; e < 4; ++e) Ls[(i * SB + kq + 4 * e) * LDL + i * SB + r] = C[e];
        fence();
    };
    // X_im = -X_ii (sum over n = m .. i-1 of L_in X_nm)
    auto inv = [&](const int i, const int m) {
        f64x4_t T = zero4, Z = zero4;
#pragma unroll
        for (int n = m; n < i; ++n)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                T = __builtin_amdgcn_mfma_f64_16x16x4f64(Ls[(i * SB + r) * LDL + n * SB + 4 * s + kq],
                                                         Xs[(n * SB + 4 * s + kq) * LDL + m * SB + r], T, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            Z = __builtin_amdgcn_mfma_f64_16x16x4f64(-Xs[(i * SB + r) * LDL + i * SB + 4 * s + kq], T[s], Z, 0, 0, 0);
        fence();
#pragma unroll
        for (int e = 0; e < 4; ++e) Xs[(i * SB + kq + 4 * e) * LDL + m * SB + r] = Z[e];
        fence();
    };
    if (w == 0) factor(0);
    __syncthreads();
    // sub-block 0: panels 1, 2, 3 (waves 0, 1, 2); then wave 0 updates and factors sub-block 1,
    // waves 1-3 update (2, 1), (2, 2); (3, 1), (3, 2); (3, 3)
    {
        f64x4_t D = zero4;
        if (w < 3) D = panel(0, 1 + w);
        __syncthreads();
        if (w == 0) {
            trail_diag(1, D);
            factor(1);
        } else if (w == 1) {
            trail(0, 2, 1);
            trail(0, 2, 2);
        } else if (w == 2) {
            trail(0, 3, 1);
            trail(0, 3, 2);
        } else {
            trail(0, 3, 3);
        }
        __syncthreads();
    }
    // sub-block 1: panels 2, 3 (waves 0, 1); wave 0: (2, 2) and the factor of sub-block 2;
    // wave 1: (3, 2); wave 2: (3, 3); wave 3: X_10
    {
        f64x4_t D = zero4;
        if (w < 2) D = panel(1, 2 + w);
        __syncthreads();
        if (w == 0) {
            trail_diag(2, D);
            factor(2);
        } else if (w == 1) {
            trail(1, 3, 2);
        } else if (w == 2) {
            trail(1, 3, 3);
        } else {
            inv(1, 0);
        }
        __syncthreads();
    }
    // sub-block 2: panel 3 (wave 0); wave 0: (3, 3) and the factor of sub-block 3;
    // wave 1: X_20; wave 2: X_21
    {
        f64x4_t D = zero4;
        if (w == 0) D = panel(2, 3);
        __syncthreads();
        if (w == 0) {
            trail_diag(3, D);
            factor(3);
        } else if (w == 1) {
            inv(2, 0);
        } else if (w == 2) {
            inv(2, 1);
        }
        __syncthreads();
    }
    // row 3 of the inverse: X_32, X_31, X_30 (waves 0, 1, 2)
    if (w < 3) inv(3, 2 - w);
    __syncthreads();
    // A pivot that is not positive and finite leaves a NaN on the factor's diagonal (the
    // reciprocal square root of a negative number, zero, infinity or NaN makes l_jj = a_jj rj
    // NaN, and the chain carries it on), so one look at the diagonal flags the system; the host
    // refuses its result.
    if (w == 0) {
        const double dg = Ls[lane * LDL + lane];
        if (!(dg > 0.0) || !isfinite(dg)) atomicOr(&g.bad[blockIdx.y], 1);
    }
    // the factor and its inverse, zero above the diagonal: to A and to Li (coalesced rows,
    // 16 per wave)
    double* Li = sys_li(g) + (size_t)kb * RB * RB;
    {
        double lv[16], xv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 16 * w + i;
            const bool low = lane <= row;
            const double lx = Ls[row * LDL + lane], xx = Xs[row * LDL + lane];
            lv[i] = low ? lx : 0.0;
            xv[i] = low ? xx : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            A[(size_t)(o + 16 * w + i) * P + o + lane] = lv[i];
            Li[(size_t)(16 * w + i) * RB + lane] = xv[i];
        }
    }
}

// C -= sum over K blocks kb = k0 .. k0 + nk - 1 of op(A) op(B), on 64 x 64 tiles with K = 64
// per block, on the fp64 matrix cores (MODE 3: C = op(A) op(B), one block, C in place).
// The tile list (i0: first row block; j0, ncol: first column block and count):
//   MODE 0  lower triangle of A:  C = A_IJ (I >= J), op(A) = A_I,kb, op(B) = A_J,kb^T.  TRI: the
//           whole lower triangle from block j0 on (lower_decode); else the rectangle
//           I in [i0, ..) x J in [j0, j0 + ncol), tiles with I < J skipped
//   MODE 2  backward update of the right-hand sides: C = Z_I,J, op(A) = L_kb,I^T, op(B) = W_kb,J
//   MODE 3  panel below block kb: C = A_I,kb (I > kb) = A_I,kb Li_kb^T
// Operand tiles are copied to LDS as they lie in memory (64 rows of 64 consecutive doubles,
// coalesced); A_ROWS / B_ROWS say whether an LDS row is an r (resp. c) index or an m index.
// 4 waves, each a 32 x 32 quarter of C as 2 x 2 blocks of 16 x 16 (v_mfma_f64_16x16x4f64:
// lane (i, k) = (lane & 15, lane >> 4) supplies A[i][k] and B[k][i]; accumulator element e
// of lane is C[(lane >> 4) + 4 e][lane & 15], rows interleaved by 4, unlike the fp32 forms).
// C is read and written once per launch, so a launch over a panel of nk blocks moves nk times
// fewer C bytes per FLOP than one launch per block.
template <int MODE, bool TRI>
__global__ __launch_bounds__(256) void ridge_update_kernel(const RidgeArgs g, int i0, int j0, int ncol, int k0,
                                                           int nk) {
    static_assert(MODE == 0 || MODE == 2 || MODE == 3, "64 x 64 update modes");
    constexpr bool A_ROWS = MODE != 2;  // LDS row of A is r (else m)
    constexpr bool B_ROWS = MODE != 2;  // LDS row of B is c (else m)
    constexpr bool OVERWRITE = MODE == 3;
    __shared__ double As[RB * LDW];
    __shared__ double Bs[RB * LDW];
    double* A = sys_a(g);
    const double* Li = sys_li(g);
    double* Bm = sys_b(g);
    const int P = g.P, Q = g.Q;
    const int tid = threadIdx.x;
    int I, J;
    if (MODE == 0 && TRI) {
        lower_decode(blockIdx.x, I, J);
        I += j0;
        J += j0;
    } else {
        I = i0 + (int)blockIdx.x / ncol;
        J = j0 + (int)blockIdx.x % ncol;
        if (MODE == 0 && I < J) return;
    }
    double* C;
    int ldc;
    if (MODE == 0 || MODE == 3) {
        C = A + (size_t)I * RB * P + (size_t)J * RB;
        ldc = P;
    } else {
        C = Bm + (size_t)I * RB * Q + (size_t)J * RB;
        ldc = Q;
    }
    const int lane = tid & 63, w = tid >> 6;
    const int r0 = (w >> 1) * 32, c0 = (w & 1) * 32;
    const int li = lane & 15, lk = lane >> 4;
    f64x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    // The operand tiles of K block k0 + kc: row x of a stored tile is at base + x * ld.
    auto tiles = [&](int kc, const double*& Ap, int& lda, const double*& Bp, int& ldb) {
        const int o = (k0 + kc) * RB;
        if (MODE == 0) {
            Ap = A + (size_t)I * RB * P + o; lda = P;   // rows r, columns m
            Bp = A + (size_t)J * RB * P + o; ldb = P;   // rows c, columns m
        } else if (MODE == 2) {
            Ap = A + (size_t)o * P + (size_t)I * RB; lda = P;   // rows m, columns r
            Bp = Bm + (size_t)o * Q + (size_t)J * RB; ldb = Q;  // rows m, columns c
        } else {
            Ap = C; lda = P;                                    // rows r, columns m
            Bp = Li + (size_t)(k0 + kc) * RB * RB; ldb = RB;    // Li rows c, columns m
        }
    };
    // Each thread moves 16 elements of each tile, consecutive threads along the unit stride;
    // the next K block's elements are loaded into registers while this one is multiplied.
    double ra[16], rb[16];
    auto fetch = [&](int kc) {
        const double* Ap;
        const double* Bp;
        int lda, ldb;
        tiles(kc, Ap, lda, Bp, ldb);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = u * 256 + tid;
            const int x = e >> 6, y = e & 63;
            ra[u] = Ap[(size_t)x * lda + y];
            rb[u] = Bp[(size_t)x * ldb + y];
        }
    };
    fetch(0);
    for (int kc = 0; kc < nk; ++kc) {
        if (kc) __syncthreads();  // every wave is done with the previous block's tiles
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = u * 256 + tid;
            const int x = e >> 6, y = e & 63;
            As[x * LDW + y] = ra[u];
            Bs[x * LDW + y] = rb[u];
        }
        __syncthreads();
        if (kc + 1 < nk) fetch(kc + 1);
        // fragments of k-step kk + 4 are read while the MFMAs of k-step kk run
        double a[2][2], b[2][2];
        auto frags = [&](int kk, int h) {
            const int m = kk + lk;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = r0 + 16 * i + li, c = c0 + 16 * i + li;
                a[h][i] = A_ROWS ? As[r * LDW + m] : As[m * LDW + r];
                b[h][i] = B_ROWS ? Bs[c * LDW + m] : Bs[m * LDW + c];
            }
        };
        frags(0, 0);
#pragma unroll
        for (int kk = 0; kk < RB; kk += 4) {
            const int h = (kk >> 2) & 1;
            if (kk + 4 < RB) frags(kk + 4, h ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // C: every element of the thread read first, then written (written element by element
    // as load-subtract-store, each load would wait for the previous store: 16 serial round trips)
    double cv[2][2][4];
    if (!OVERWRITE) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    cv[i][j][e] = C[(size_t)(r0 + 16 * i + lk + 4 * e) * ldc + c0 + 16 * j + li];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + 16 * i + lk + 4 * e, c = c0 + 16 * j + li;
                C[(size_t)r * ldc + c] = OVERWRITE ? acc[i][j][e] : cv[i][j][e] - acc[i][j][e];
            }
}

// Substitution inside one panel of nbk blocks from b0, one workgroup per CW columns J of the
// right-hand sides (the rows outside the panel already updated by every earlier panel):
//   forward  (L Z = B):    for kb = b0 .. b0 + nbk - 1:  Z_kb = Li_kb B_kb,    then B_I -= L_I,kb Z_kb  (I in (kb, b0 + nbk))
//   backward (L^T W = Z):  for kb = b0 + nbk - 1 .. b0:  W_kb = Li_kb^T Z_kb,  then Z_I -= L_kb,I^T W_kb  (I in [b0, kb))
// A column block's chain needs no other column block, so the whole chain of a panel is one
// launch (it had been two launches per block).  The panel's blocks of the right-hand sides stay
// in registers (accumulator layout, 16 values per block and thread); each product's operand
// (Li_kb or a 64 x 64 block of L) is read into registers during the previous product and goes
// through a two-deep LDS ring; the diagonal step's input and result go through LDS as the B
// operand.  4 waves, each a 32 x CW/2 quarter of the 64 x CW block as 2 x CW/32 blocks of
// 16 x 16 (v_mfma_f64_16x16x4f64, accumulator element e of a lane at row (lane >> 4) + 4 e).
template <bool BACK, int CW>
__global__ __launch_bounds__(256) void ridge_panel_subst_kernel(const RidgeArgs g, int b0, int nbk) {
    constexpr int MAXB = 4;  // blocks per panel
    constexpr int NJ = CW / 32;  // 16-wide column blocks per wave (CW columns per workgroup)
    __shared__ double Os[2][RB * LDW];  // operand ring: Os[x][y] = O[x][y], O = Li_kb or a block of L
    __shared__ double Zs[RB * LDW];     // the diagonal step's input, then
    __shared__ double Ws[RB * LDW];     // its result
    const double* A = sys_a(g);
    const double* Li = sys_li(g);
    double* Bm = sys_b(g);
    const int P = g.P, Q = g.Q;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r0 = (w >> 1) * 32, c0 = (w & 1) * (CW / 2);
    const int li = lane & 15, lk = lane >> 4;
    const int J = (int)blockIdx.x;
    f64x4_t z[MAXB][2][NJ];
#pragma unroll
    for (int t = 0; t < MAXB; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    z[t][i][j][e] = (t < nbk) ? Bm[(size_t)((b0 + t) * RB + r0 + 16 * i + lk + 4 * e) * Q + J * CW + c0 + 16 * j + li]
                                              : 0.0;
    // the operand of product (t, u): Li_kb (u < 0) or, for the update of row block I = b0 + u,
    // L_kb,I (backward) or L_I,kb (forward), kb = b0 + t
    double ro[16];
    auto fetch = [&](int t, int u) {
        const int kb = b0 + t, I = b0 + u;
        const double* src = (u < 0) ? Li + (size_t)kb * RB * RB
                            : BACK  ? A + (size_t)kb * RB * P + (size_t)I * RB
                                    : A + (size_t)I * RB * P + (size_t)kb * RB;
        const int ld = (u < 0) ? RB : P;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int e = v * 256 + tid;
            ro[v] = src[(size_t)(e >> 6) * ld + (e & 63)];
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int e = v * 256 + tid;
            Os[buf][(e >> 6) * LDW + (e & 63)] = ro[v];
        }
    };
    // acc (+/-)= op(O) X, op(O) = O^T (backward) or O (forward), X from LDS
    auto product = [&](f64x4_t (&acc)[2][NJ], const double* os, const double* xs, bool neg) {
#pragma unroll
        for (int kk = 0; kk < RB; kk += 4) {
            const int m = kk + lk;
            double a[2], b[NJ];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = r0 + 16 * i + li;
                const double v = BACK ? os[m * LDW + r] : os[r * LDW + m];
                a[i] = neg ? -v : v;
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = xs[m * LDW + c0 + 16 * j + li];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    auto put = [&](double* xs, const f64x4_t (&v)[2][NJ]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[(r0 + 16 * i + lk + 4 * e) * LDW + c0 + 16 * j + li] = v[i][j][e];
    };
    // products in order: for each diagonal step t (backward: from the last), (t, -1), then the
    // updates (t, u) of the panel's row blocks u still to come
    auto upd_ok = [&](int t, int u) { return BACK ? (u < t) : (u > t && u < nbk); };
    int q = 0;
    fetch(BACK ? nbk - 1 : 0, -1);
#pragma unroll
    for (int tt = 0; tt < MAXB; ++tt) {
        const int t = BACK ? MAXB - 1 - tt : tt;
        if (t >= nbk) continue;
#pragma unroll
        for (int u = -1; u < MAXB; ++u) {
            if (u >= 0 && !upd_ok(t, u)) continue;
            const int buf = q & 1;
            stash(buf);  // that buffer's last reader was product q - 2, before the last barrier
            if (u < 0) put(Zs, z[t]);
            // the next product's operand
            {
                int nu = u + 1;
                while (nu < MAXB && !upd_ok(t, nu)) ++nu;
                if (nu < MAXB) fetch(t, nu);
                else if (BACK ? t > 0 : t + 1 < nbk) fetch(BACK ? t - 1 : t + 1, -1);
            }
            __syncthreads();
            if (u < 0) {
                f64x4_t acc[2][NJ];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
                product(acc, Os[buf], Zs, false);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) z[t][i][j] = acc[i][j];
                put(Ws, z[t]);  // Ws's last readers were the previous step's updates, before the barrier
            } else {
                product(z[u], Os[buf], Ws, true);
            }
            ++q;
        }
    }
#pragma unroll
    for (int t = 0; t < MAXB; ++t)
        if (t < nbk) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Bm[(size_t)((b0 + t) * RB + r0 + 16 * i + lk + 4 * e) * Q + J * CW + c0 + 16 * j + li] = z[t][i][j][e];
        }
}

// The large updates of MODE 0 (TRI), 1 and 2 of ridge_update_kernel on 128 x 128 tiles of C, K
// = 64 nk from block k0 (i0, j0: first row and column tile, in tiles of 128; ncol: column tiles;
// MODE 0 takes the lower triangle of tiles from tile j0 on, and computes the diagonal tiles
// whole: their upper 64 x 64 quarter is never read).  Twice the arithmetic per operand byte of
// the 64 x 64 kernel.  8 waves, each a 64 x 32 eighth of C as 4 x 2 blocks of 16 x 16
// (v_mfma_f64_16x16x4f64).  The operands go through LDS in stages of K = KB, two stages
// deep: the registers holding stage kc + 1 are written to LDS, and stage kc + 2 is requested,
// before the MFMAs of stage kc, so neither waits on the other.  KB = 32 takes 132-135 KiB of
// LDS, one workgroup per CU; KB = 16 takes 66-68 KiB, two per CU, so that one workgroup's C
// epilogue overlaps the other's products (faster for batches of systems and for the back
// substitution; for one system's factorisation and forward substitution, beside which its
// serial chain of small kernels runs, KB = 32 measured faster).
template <int MODE, int KB>
__global__ __launch_bounds__(512) void ridge_big_kernel(const RidgeArgs g, int i0, int j0, int ncol, int k0,
                                                        int nk) {
    static_assert(MODE == 0 || MODE == 1 || MODE == 2, "large-update modes");
    constexpr int LD_R = KB + 1;  // LDS row stride of a stage stored with the tile's rows (128 x KB)
    constexpr bool A_ROWS = MODE != 2;  // A stage stored with the rows r (else with m as rows)
    constexpr bool B_ROWS = MODE == 0;  // B stage stored with the columns c as rows (else m)
    constexpr int A_LDS = A_ROWS ? TB * LD_R : KB * LD_M;
    constexpr int B_LDS = B_ROWS ? TB * LD_R : KB * LD_M;
    __shared__ double As[2][A_LDS];
    __shared__ double Bs[2][B_LDS];
    double* A = sys_a(g);
    double* Bm = sys_b(g);
    const int P = g.P, Q = g.Q;
    const int tid = threadIdx.x;
    int I, J;
    if (MODE == 0) {
        lower_decode(blockIdx.x, I, J);
        I += j0;
        J += j0;
    } else {
        I = i0 + (int)blockIdx.x / ncol;
        J = j0 + (int)blockIdx.x % ncol;
    }
    double* C;
    int ldc;
    if (MODE == 0) {
        C = A + (size_t)I * TB * P + (size_t)J * TB;
        ldc = P;
    } else {
        C = Bm + (size_t)I * TB * Q + (size_t)J * TB;
        ldc = Q;
    }
    // stage kc: element (x, y) of the stored A (B) stage is Ap[x * lda + y] (Bp[x * ldb + y])
    auto stage = [&](int kc, const double*& Ap, int& lda, const double*& Bp, int& ldb) {
        const int ko = k0 * RB + kc * KB;
        if (MODE == 0) {
            Ap = A + (size_t)I * TB * P + ko; lda = P;  // rows r, columns m
            Bp = A + (size_t)J * TB * P + ko; ldb = P;  // rows c, columns m
        } else if (MODE == 1) {
            Ap = A + (size_t)I * TB * P + ko; lda = P;  // rows r, columns m
            Bp = Bm + (size_t)ko * Q + (size_t)J * TB; ldb = Q;  // rows m, columns c
        } else {
            Ap = A + (size_t)ko * P + (size_t)I * TB; lda = P;  // rows m, columns r
            Bp = Bm + (size_t)ko * Q + (size_t)J * TB; ldb = Q;  // rows m, columns c
        }
    };
    constexpr int PER = TB * KB / 512;  // elements of each stage per thread (8 at KB = 32)
    double ra[PER], rb[PER];
    auto fetch = [&](int kc) {
        const double* Ap;
        const double* Bp;
        int lda, ldb;
        stage(kc, Ap, lda, Bp, ldb);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = u * 512 + tid;
            const int xa = A_ROWS ? e / KB : e / TB, ya = A_ROWS ? e % KB : e % TB;
            const int xb = B_ROWS ? e / KB : e / TB, yb = B_ROWS ? e % KB : e % TB;
            ra[u] = Ap[(size_t)xa * lda + ya];
            rb[u] = Bp[(size_t)xb * ldb + yb];
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = u * 512 + tid;
            const int xa = A_ROWS ? e / KB : e / TB, ya = A_ROWS ? e % KB : e % TB;
            const int xb = B_ROWS ? e / KB : e / TB, yb = B_ROWS ? e % KB : e % TB;
            As[buf][xa * (A_ROWS ? LD_R : LD_M) + ya] = ra[u];
            Bs[buf][xb * (B_ROWS ? LD_R : LD_M) + yb] = rb[u];
        }
    };
    const int lane = tid & 63, w = tid >> 6;
    const int wr0 = (w >> 2) * 64, wc0 = (w & 3) * 32;
    const int li = lane & 15, lk = lane >> 4;
    f64x4_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    static_assert((RB / KB) % 2 == 0, "stages come in pairs");
    const int nkb = nk * (RB / KB);
    fetch(0);
    stash(0);
    if (nkb > 1) fetch(1);
    __syncthreads();
    // one stage; cur is a constant in both calls below, so every LDS address folds
    auto kstage = [&](int kc, const int cur) {
        if (kc + 1 < nkb) stash(cur ^ 1);  // that buffer's last reader was stage kc - 1
        if (kc + 2 < nkb) fetch(kc + 2);
        const double* as = As[cur];
        const double* bs = Bs[cur];
#pragma unroll
        for (int kk = 0; kk < KB; kk += 4) {
            const int m = kk + lk;
            double a[4], b[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wr0 + 16 * i + li;
                a[i] = A_ROWS ? as[r * LD_R + m] : as[m * LD_M + r];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = wc0 + 16 * j + li;
                b[j] = B_ROWS ? bs[c * LD_R + m] : bs[m * LD_M + c];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();  // stage kc read by every wave before its buffer is refilled
    };
    for (int kc = 0; kc < nkb; kc += 2) {  // nkb = nk RB / KB is even
        kstage(kc, 0);
        kstage(kc + 1, 1);
    }
    double cv[4][2][4];  // C read whole before any store (see ridge_update_kernel)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) cv[i][j][e] = C[(size_t)(wr0 + 16 * i + lk + 4 * e) * ldc + wc0 + 16 * j + li];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = wr0 + 16 * i + lk + 4 * e, c = wc0 + 16 * j + li;
                C[(size_t)r * ldc + c] = cv[i][j][e] - acc[i][j][e];
            }
}

// W_out[c][i] = W[i][c] in the output dtype (output-major): one 64 x 64 tile per workgroup,
// through LDS, so rows of W are read and rows of W_out written as coalesced runs.
template <bool BF16>
__global__ __launch_bounds__(256) void ridge_out_kernel(const RidgeArgs g) {
    __shared__ double t[RB][RB + 1];
    const RidgeSys& S = g.s[blockIdx.y];
    const double* W = sys_b(g);
    const int Q = g.Q, p = g.p, q = g.q;
    const int i0 = (int)blockIdx.x * RB, c0 = (int)blockIdx.z * RB;  // grid: (row tiles, system, column tiles)
    const int tid = threadIdx.x, cx = tid & 63, ry = tid >> 6;
    for (int rr = ry; rr < RB; rr += 4) {
        const int i = i0 + rr;
        t[rr][cx] = (i < p) ? W[(size_t)i * Q + c0 + cx] : 0.0;
    }
    __syncthreads();
    for (int cc = ry; cc < RB; cc += 4) {
        const int c = c0 + cc, i = i0 + cx;
        if (c < q && i < p) {
            const double v = t[cx][cc];
            if (BF16) ((uint16_t*)S.W_out)[(size_t)c * p + i] = (uint16_t)(pack_bf16((float)v, 0.f) & 0xffffu);
            else ((float*)S.W_out)[(size_t)c * p + i] = (float)v;
        }
    }
}

// b[c] = mean_y[c] - sum_i mean_x[i] W[i][c] (fp64).  Workgroup: 16 columns x 16 row groups
// (a wave reads 4 rows of 16 consecutive doubles, whole 128-byte lines); the row groups are
// added in a fixed order.
template <bool BF16>
__global__ __launch_bounds__(256) void ridge_bias_kernel(const RidgeArgs g) {
    constexpr int BC = 16, RG = 16;
    __shared__ double part[RG][BC + 1];
    const RidgeSys& S = g.s[blockIdx.y];
    const double* W = sys_b(g);
    const int Q = g.Q, p = g.p, q = g.q;
    const int tid = threadIdx.x, cx = tid % BC, ry = tid / BC;
    const int c = (int)blockIdx.x * BC + cx;
    double dot = 0.0;
    if (c < q) {
#pragma unroll 8
        for (int i = ry; i < p; i += RG) dot += (double)S.mean_x[i] * W[(size_t)i * Q + c];
    }
    part[ry][cx] = dot;
    __syncthreads();
    if (ry == 0 && c < q) {
        double sum = 0.0;
        for (int r = 0; r < RG; ++r) sum += part[r][cx];
        const double bv = (double)S.mean_y[c] - sum;
        if (BF16) ((uint16_t*)S.b_out)[c] = (uint16_t)(pack_bf16((float)bv, 0.f) & 0xffffu);
        else ((float*)S.b_out)[c] = (float)bv;
    }
}

// In-sample residual sum of squares of column c from the statistics alone.  With
// yc = y - mean_y, xc = x - mean_x and (M_xx + lambda I) w = m (m = M_xy[:, c]):
//   sum (yc - xc w)^2 = ss_y[c] - 2 w.m + w^T M_xx w = ss_y[c] - w.m - lambda |w|^2,
// since w^T M_xx w = w^T (m - lambda w).  Workgroup: 64 columns; the 4 row groups are
// reduced in a fixed order.
__global__ __launch_bounds__(256) void ridge_rss_kernel(const RidgeArgs g) {
    __shared__ double pd[4][RB];
    __shared__ double pn[4][RB];
    const RidgeSys& S = g.s[blockIdx.y];
    const double* W = sys_b(g);
    const int Q = g.Q, p = g.p, q = g.q;
    const int tid = threadIdx.x;
    const int cx = tid & 63, ry = tid >> 6;
    const int c = (int)blockIdx.x * RB + cx;
    double dot = 0.0, nrm = 0.0;
    if (c < q) {
        for (int i = ry; i < p; i += 4) {
            const double w = W[(size_t)i * Q + c];
            dot += w * (double)S.M_xy[(size_t)i * q + c];
            nrm += w * w;
        }
    }
    pd[ry][cx] = dot;
    pn[ry][cx] = nrm;
    __syncthreads();
    if (ry == 0 && c < q) {
        const double d = ((pd[0][cx] + pd[1][cx]) + pd[2][cx]) + pd[3][cx];
        const double n2 = ((pn[0][cx] + pn[1][cx]) + pn[2][cx]) + pn[3][cx];
        sys_rss(g)[c] = (double)S.ss_y[c] - d - g.lambda * n2;
    }
}

// R^2 of group gi (columns gi*group .. gi*group + group - 1) pooled over its columns:
// 1 - sum RSS / sum ss_y; NaN when the group's total sum of squares is 0.
__global__ __launch_bounds__(256) void ridge_r2_group_kernel(const RidgeArgs g, int group) {
    const int groups = g.q / group;
    const int gi = (int)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi >= groups) return;
    const RidgeSys& S = g.s[blockIdx.y];
    const double* rss = sys_rss(g);
    double r = 0.0, t = 0.0;
    for (int j = 0; j < group; ++j) {
        r += rss[(size_t)gi * group + j];
        t += (double)S.ss_y[(size_t)gi * group + j];
    }
    S.r2_out[gi] = t > 0.0 ? 1.0 - r / t : __builtin_nan("");
}

// ---------------------------------------------------------------------------------------

namespace {

// P, Q: p and q padded to a multiple of the 128-wide tiles of the large updates (so that every
// panel boundary, a multiple of 4 blocks of 64, is a tile boundary).
int pad_dim(int n) { return (n + TB - 1) / TB * TB; }

size_t sys_stride(int p, int q) {
    const size_t P = (size_t)pad_dim(p), Q = (size_t)pad_dim(q);
    return (P * P + P * Q + Q + P * RB + 31) / 32 * 32;  // A, B (then W), rss, Li; 256-byte aligned
}

RidgeArgs make_args(int n, int p, int q, const RidgeSys* sys, double lambda, void* scratch) {
    RidgeArgs g{};
    for (int i = 0; i < n; ++i) g.s[i] = sys[i];
    g.scratch = (double*)scratch;
    g.stride = sys_stride(p, q);
    g.bad = ridge_dev_flags(scratch, p, q, n);
    g.p = p;
    g.q = q;
    g.P = pad_dim(p);
    g.Q = pad_dim(q);
    g.lambda = lambda;
    return g;
}

// A = L L^T (lower triangle of A), then W = A^-1 M_xy in B, row-major [P][Q], every system.
// The 64-wide blocks are taken in panels of kPanel: inside a panel each block is factored and
// applied to the panel's own columns (and, in the substitutions, its own rows) at once; the
// rest of the matrix (or of the right-hand sides) is updated once per panel with K = 64 kPanel.
constexpr int kPanel = 4;
static_assert(kPanel <= 4, "ridge_panel_subst_kernel holds at most 4 blocks in registers");
// The substitutions inside a panel: 32 columns of the right-hand sides per workgroup for one
// system (twice the workgroups on the serial chain), 64 for a batch (fewer operand reloads)
template <bool BACK>
void launch_subst(const RidgeArgs& g, unsigned un, int b0, int nbk, hipStream_t s) {
    if (un > 1) hipLaunchKernelGGL((ridge_panel_subst_kernel<BACK, 64>), dim3(g.Q / 64, un), dim3(256), 0, s, g, b0, nbk);
    else hipLaunchKernelGGL((ridge_panel_subst_kernel<BACK, 32>), dim3(g.Q / 32, un), dim3(256), 0, s, g, b0, nbk);
}

// A large update: stages of K = 16 (two workgroups per CU) for a batch of systems and for the
// back substitution, 32 for the factorisation and forward substitution of one system
template <int MODE>
void launch_big(dim3 grid, hipStream_t s, const RidgeArgs& g, int i0, int j0, int ncol, int k0, int nk) {
    if (grid.y > 1 || MODE == 2) hipLaunchKernelGGL((ridge_big_kernel<MODE, 16>), grid, dim3(512), 0, s, g, i0, j0, ncol, k0, nk);
    else hipLaunchKernelGGL((ridge_big_kernel<MODE, 32>), grid, dim3(512), 0, s, g, i0, j0, ncol, k0, nk);
}

// Forward substitution over the panel [b0, b1): the chain inside the panel (each diagonal step a
// product with the block's inverse) in one launch, then the rows below the panel updated once
// with K = the panel.  Reads only the
// factored panel (its columns of L and its blocks' inverses) and writes B.
static void forward_panel(const RidgeArgs& g, int n, int b0, hipStream_t s) {
    const int nb = g.P / RB, nq2 = g.Q / TB;
    const unsigned un = (unsigned)n;
    const int b1 = std::min(nb, b0 + kPanel);
    launch_subst<false>(g, un, b0, b1 - b0, s);
    if (nb > b1)
        launch_big<1>(dim3((nb - b1) / 2 * nq2, un), s, g, b1 / 2, 0, nq2, b0, b1 - b0);
}

void solve_batch(const RidgeArgs& g, int n, hipStream_t s, const RidgeOverlap& ov) {
    const int P = g.P, Q = g.Q;
    const int nb = P / RB, nq = Q / RB, nq2 = Q / TB;  // (P, Q: multiples of 128, so nb is even and every
                                                        // panel boundary, a multiple of 4 blocks, is even)
    const unsigned un = (unsigned)n;
    const dim3 blk(256);
    hipLaunchKernelGGL(ridge_init_a_kernel, dim3((unsigned)(nb * (nb + 1) / 2), un), blk, 0, s, g);
    hipLaunchKernelGGL(ridge_init_b_kernel, dim3((unsigned)(((int64_t)P * Q + 255) / 256), un), blk, 0, s, g);
    // Factorisation with a one-panel lookahead.  After panel [b0, b1) is factored, its update of
    // the next panel's columns [b1, b2) (rows b1 ..) runs on `s`, and its update of the rest of
    // the trailing triangle (rows and columns b2 ..) on the side stream, where it overlaps the
    // next panel's serial chain of diagonal steps (which touch only columns [b1, b2)).  The next
    // lookahead update writes columns that the side update writes too, so `s` waits for it first.
    // Without a side stream (ov.side NULL) the whole trailing update runs on `s`.  With a forward
    // stream, each factored panel's forward substitution (it reads only that panel's columns of L
    // and writes B) runs there as soon as the panel is done.
    bool side_pending = false;
    for (int b0 = 0; b0 < nb; b0 += kPanel) {
        const int b1 = std::min(nb, b0 + kPanel);
        for (int kb = b0; kb < b1; ++kb) {
            hipLaunchKernelGGL(ridge_potrf_kernel, dim3(1, un), dim3(256), 0, s, g, kb);
            const int below = nb - kb - 1;
            if (below == 0) continue;
            hipLaunchKernelGGL((ridge_update_kernel<3, false>), dim3(below, un), blk, 0, s, g, kb + 1, kb, 1, kb, 1);
            const int w = b1 - kb - 1;  // the panel's columns right of kb, every row below
            if (w > 0)
                hipLaunchKernelGGL((ridge_update_kernel<0, false>), dim3(below * w, un), blk, 0, s, g, kb + 1, kb + 1,
                                   w, kb, 1);
        }
        if (ov.fwd) {  // this panel's forward substitution, on the forward stream
            (void)hipEventRecord(ov.fwd_ready, s);
            (void)hipStreamWaitEvent(ov.fwd, ov.fwd_ready, 0);
            forward_panel(g, n, b0, ov.fwd);
        }
        if (b1 == nb) break;
        if (!ov.side) {
            const int m = (nb - b1) / 2;  // trailing lower triangle, in tiles of 128
            launch_big<0>(dim3(m * (m + 1) / 2, un), s, g, 0, b1 / 2, 0, b0, b1 - b0);
            continue;
        }
        const int b2 = std::min(nb, b1 + kPanel);
        if (side_pending) (void)hipStreamWaitEvent(s, ov.side_done, 0);
        // lookahead: tiles (I, J) of 64, I in [b1, nb), J in [b1, b2), I >= J, K = the panel
        hipLaunchKernelGGL((ridge_update_kernel<0, false>), dim3((nb - b1) * (b2 - b1), un), blk, 0, s, g, b1, b1,
                           b2 - b1, b0, b1 - b0);
        side_pending = false;
        if (b2 == nb) continue;
        const int m = (nb - b2) / 2;  // the rest: lower triangle of 128-tiles from b2
        (void)hipEventRecord(ov.main_ready, s);
        (void)hipStreamWaitEvent(ov.side, ov.main_ready, 0);
        launch_big<0>(dim3(m * (m + 1) / 2, un), ov.side, g, 0, b2 / 2, 0, b0, b1 - b0);
        (void)hipEventRecord(ov.side_done, ov.side);
        side_pending = true;
    }
    if (side_pending) (void)hipStreamWaitEvent(s, ov.side_done, 0);
    if (ov.fwd) {
        (void)hipEventRecord(ov.fwd_done, ov.fwd);
        (void)hipStreamWaitEvent(s, ov.fwd_done, 0);
    }
    // L Z = B (here only without the forward stream; with it, each panel ran on that stream
    // right after the panel was factored)
    if (!ov.fwd)
        for (int b0 = 0; b0 < nb; b0 += kPanel) forward_panel(g, n, b0, s);
    // L^T W = Z, panels from the last, with a two-panel lookahead.  Panel k, counted from the
    // end, is blocks [s_k, e_k).  Once panel k is solved, the caller's stream updates the rows of
    // panel k + 1 with panels k - 1 and k (K up to 8 blocks), so that panel's chain can start,
    // and the side stream updates the rows above panel k + 2, [0, s_(k+2)), with panel k.  The
    // streams then never write the same rows at once: panel k + 1's rows were last written on
    // the side stream by the update of panel k - 2, which the lookahead waits for (two events in
    // turn, so that it does not wait for the side update just queued).
    std::vector<std::pair<int, int>> pan;  // (s_k, e_k)
    for (int e = nb; e > 0; e -= kPanel) pan.push_back({std::max(0, e - kPanel), e});
    const int np = (int)pan.size();
    const hipEvent_t done[2] = {ov.side_done, ov.side_done2};
    bool pending[2] = {false, false};
    for (int k = 0; k < np; ++k) {
        const int sk = pan[k].first, ek = pan[k].second;
        launch_subst<true>(g, un, sk, ek - sk, s);
        if (k + 1 == np) break;
        if (!ov.side) {
            launch_big<2>(dim3(sk / 2 * nq2, un), s, g, 0, 0, nq2, sk, ek - sk);
            continue;
        }
        if (pending[k % 2]) {  // the side update of panel k - 2
            (void)hipStreamWaitEvent(s, done[k % 2], 0);
            pending[k % 2] = false;
        }
        const int kend = k > 0 ? pan[k - 1].second : ek;  // panels k - 1 and k
        const int rs = pan[k + 1].first, re = pan[k + 1].second;
        hipLaunchKernelGGL((ridge_update_kernel<2, false>), dim3((re - rs) * nq, un), blk, 0, s, g, rs, 0, nq, sk,
                           kend - sk);
        const int top = k + 2 < np ? pan[k + 2].first : 0;
        if (top == 0) continue;
        (void)hipEventRecord(ov.main_ready, s);
        (void)hipStreamWaitEvent(ov.side, ov.main_ready, 0);
        launch_big<2>(dim3(top / 2 * nq2, un), ov.side, g, 0, 0, nq2, sk, ek - sk);
        (void)hipEventRecord(done[k % 2], ov.side);
        pending[k % 2] = true;
    }
    for (int i = 0; i < 2; ++i)
        if (pending[i]) (void)hipStreamWaitEvent(s, done[i], 0);
}

}  // namespace

size_t ridge_dev_scratch_bytes(int p, int q, int n) { return (size_t)n * sys_stride(p, q) * sizeof(double) + 256; }

int* ridge_dev_flags(void* scratch, int p, int q, int n) {
    return (int*)((char*)scratch + (size_t)n * sys_stride(p, q) * sizeof(double));
}

hipError_t launch_ridge_dev(int n, int p, int q, const RidgeSys* sys, double lambda, bool bf16, void* scratch,
                            hipStream_t s, const RidgeOverlap& ov) {
    if (n < 1 || n > kRidgeMaxBatch) return hipErrorInvalidValue;
    const RidgeArgs g = make_args(n, p, q, sys, lambda, scratch);
    solve_batch(g, n, s, ov);
    const dim3 tiles((unsigned)((p + RB - 1) / RB), (unsigned)n, (unsigned)(g.Q / RB));  // system on grid y
    const dim3 cols((unsigned)((q + 15) / 16), (unsigned)n);
    if (bf16) {
        hipLaunchKernelGGL(ridge_out_kernel<true>, tiles, dim3(256), 0, s, g);
        hipLaunchKernelGGL(ridge_bias_kernel<true>, cols, dim3(256), 0, s, g);
    } else {
        hipLaunchKernelGGL(ridge_out_kernel<false>, tiles, dim3(256), 0, s, g);
        hipLaunchKernelGGL(ridge_bias_kernel<false>, cols, dim3(256), 0, s, g);
    }
    return hipGetLastError();
}

hipError_t launch_ridge_r2(int n, int p, int q, const RidgeSys* sys, double lambda, int group, void* scratch,
                           hipStream_t s, const RidgeOverlap& ov) {
    if (n < 1 || n > kRidgeMaxBatch || group < 1 || q % group) return hipErrorInvalidValue;
    const RidgeArgs g = make_args(n, p, q, sys, lambda, scratch);
    solve_batch(g, n, s, ov);
    hipLaunchKernelGGL(ridge_rss_kernel, dim3(g.Q / RB, (unsigned)n), dim3(256), 0, s, g);
    const int groups = q / group;
    hipLaunchKernelGGL(ridge_r2_group_kernel, dim3((groups + 255) / 256, (unsigned)n), dim3(256), 0, s, g, group);
    return hipGetLastError();
}

}  // namespace kvmap
