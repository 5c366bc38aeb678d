// Closed-form ridge on the host in float64 (KVBridge README, fitting section headed
// "Loading": W = (X^T X + lambda I)^-1 X^T Y, b = Ybar - Xbar W; reactapp.top article, section
// "Eine lineare Bruecke reicht": lambda = 0.01 added to the centred Gram, intercept from the
// means, so the intercept is not penalised).
//
//   A = sym(M_xx) + lambda I = L L^T          blocked right-looking Cholesky
//   L Z = M_xy,  L^T W = Z                    blocked over right-hand-side columns
//   b = mean_y - mean_x W
//
// Threads: the trailing update of each Cholesky step is split into 64x64 tiles of the
// lower triangle handed out through an atomic counter; the two triangular solves are split
// over chunks of right-hand-side columns (each chunk's Z stays cache resident).

#include "ridge.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <thread>
#include <vector>

namespace kvmap {

namespace {

template <typename Fn>
void parallel_for(int n_items, int n_threads, Fn fn) {
    if (n_items <= 0) return;
    const int nt = std::max(1, std::min(n_threads, n_items));
    if (nt == 1) {
        for (int i = 0; i < n_items; ++i) fn(i);
        return;
    }
    std::atomic<int> next{0};
    std::vector<std::thread> pool;
    pool.reserve(nt);
    for (int t = 0; t < nt; ++t)
        pool.emplace_back([&] {
            for (int i = next.fetch_add(1); i < n_items; i = next.fetch_add(1)) fn(i);
        });
    for (auto& th : pool) th.join();
}

constexpr int NB = 96;   // Cholesky panel width
constexpr int TB = 64;   // trailing-update tile
constexpr int RC = 32;   // right-hand-side columns per solve chunk

// C[i][j] -= sum_m P[i][m] P[j][m] over a TB x TB tile of the trailing lower triangle.
// P is the packed panel [rows][b] (row-major), C the full matrix with leading dim ld.
void syrk_tile(double* C, int ld, const double* P, int b, int i0, int i1, int j0, int j1,
               int off) {
    for (int i = i0; i < i1; i += 4) {
        const int ni = std::min(4, i1 - i);
        for (int j = j0; j < j1 && j <= i + 3; j += 4) {
            const int nj = std::min(4, j1 - j);
            double acc[4][4] = {};
            const double* pi[4];
            const double* pj[4];
            for (int a = 0; a < 4; ++a) {
                pi[a] = P + (size_t)(std::min(i + a, i1 - 1) - off) * b;
                pj[a] = P + (size_t)(std::min(j + a, j1 - 1) - off) * b;
            }
            for (int m = 0; m < b; ++m) {
                const double x0 = pi[0][m], x1 = pi[1][m], x2 = pi[2][m], x3 = pi[3][m];
                const double y0 = pj[0][m], y1 = pj[1][m], y2 = pj[2][m], y3 = pj[3][m];
                acc[0][0] += x0 * y0; acc[0][1] += x0 * y1; acc[0][2] += x0 * y2; acc[0][3] += x0 * y3;
                acc[1][0] += x1 * y0; acc[1][1] += x1 * y1; acc[1][2] += x1 * y2; acc[1][3] += x1 * y3;
                acc[2][0] += x2 * y0; acc[2][1] += x2 * y1; acc[2][2] += x2 * y2; acc[2][3] += x2 * y3;
                acc[3][0] += x3 * y0; acc[3][1] += x3 * y1; acc[3][2] += x3 * y2; acc[3][3] += x3 * y3;
            }
            for (int a = 0; a < ni; ++a)
                for (int c = 0; c < nj; ++c)
                    if (j + c <= i + a) C[(size_t)(i + a) * ld + (j + c)] -= acc[a][c];
        }
    }
}

}  // namespace

int ridge_solve_f64(int p, int q, const float* mean_x, const float* mean_y, const float* M_xx,
                    const float* M_xy, double lambda, float* W_out, float* b_out,
                    int n_threads) {
    if (n_threads <= 0) n_threads = (int)std::max(1u, std::thread::hardware_concurrency());
    const size_t P = (size_t)p;
    // Lower triangle of A from the upper triangle of M_xx, plus lambda on the diagonal.
    std::vector<double> A(P * P, 0.0);
    parallel_for(p, n_threads, [&](int i) {
        for (int j = 0; j <= i; ++j) A[(size_t)i * P + j] = (double)M_xx[(size_t)j * P + i];
        A[(size_t)i * P + i] += lambda;
    });

    std::vector<double> panel;
    std::atomic<int> bad{0};
    for (int k = 0; k < p; k += NB) {
        const int b = std::min(NB, p - k);
        // 1. diagonal block, unblocked
        for (int j = k; j < k + b; ++j) {
            double s = A[(size_t)j * P + j];
            for (int m = k; m < j; ++m) s -= A[(size_t)j * P + m] * A[(size_t)j * P + m];
            if (!(s > 0.0)) return 1;
            const double d = std::sqrt(s);
            A[(size_t)j * P + j] = d;
            for (int i = j + 1; i < k + b; ++i) {
                double t = A[(size_t)i * P + j];
                for (int m = k; m < j; ++m) t -= A[(size_t)i * P + m] * A[(size_t)j * P + m];
                A[(size_t)i * P + j] = t / d;
            }
        }
        const int r0 = k + b, nr = p - r0;
        if (nr <= 0) break;
        // 2. panel rows below: row_i <- row_i L_kk^-T, packed into `panel`
        panel.assign((size_t)nr * b, 0.0);
        parallel_for((nr + 63) / 64, n_threads, [&](int blk) {
            for (int i = r0 + blk * 64; i < std::min(p, r0 + blk * 64 + 64); ++i) {
                double* row = &A[(size_t)i * P + k];
                for (int j = 0; j < b; ++j) {
                    double t = row[j];
                    const double* lj = &A[(size_t)(k + j) * P + k];
                    for (int m = 0; m < j; ++m) t -= row[m] * lj[m];
                    row[j] = t / lj[j];
                }
                std::copy(row, row + b, &panel[(size_t)(i - r0) * b]);
            }
        });
        // 3. trailing update of the lower triangle in TB x TB tiles
        const int nt = (nr + TB - 1) / TB;
        const int ntiles = nt * (nt + 1) / 2;
        parallel_for(ntiles, n_threads, [&](int u) {
            int ti = 0;
            while ((ti + 1) * (ti + 2) / 2 <= u) ++ti;
            const int tj = u - ti * (ti + 1) / 2;
            const int i0 = r0 + ti * TB, i1 = std::min(p, i0 + TB);
            const int j0 = r0 + tj * TB, j1 = std::min(p, j0 + TB);
            syrk_tile(A.data(), p, panel.data(), b, i0, i1, j0, j1, r0);
        });
    }
    (void)bad;

    // Triangular solves over chunks of RC right-hand-side columns.
    std::vector<double> W(P * (size_t)q);
    const int nchunks = (q + RC - 1) / RC;
    parallel_for(nchunks, n_threads, [&](int ch) {
        const int c0 = ch * RC, nc = std::min(RC, q - c0);
        std::vector<double> Z(P * RC, 0.0);
        for (int i = 0; i < p; ++i)
            for (int c = 0; c < nc; ++c) Z[(size_t)i * RC + c] = (double)M_xy[(size_t)i * q + c0 + c];
        // forward: L Z = B  (dot form over rows of L)
        for (int i = 0; i < p; ++i) {
            double acc[RC];
            for (int c = 0; c < RC; ++c) acc[c] = Z[(size_t)i * RC + c];
            const double* li = &A[(size_t)i * P];
            for (int m = 0; m < i; ++m) {
                const double l = li[m];
                const double* zm = &Z[(size_t)m * RC];
                for (int c = 0; c < RC; ++c) acc[c] -= l * zm[c];
            }
            const double inv = 1.0 / li[i];
            for (int c = 0; c < RC; ++c) Z[(size_t)i * RC + c] = acc[c] * inv;
        }
        // backward: L^T W = Z  (axpy form over rows of L)
        for (int i = p - 1; i >= 0; --i) {
            const double* li = &A[(size_t)i * P];
            double* zi = &Z[(size_t)i * RC];
            const double inv = 1.0 / li[i];
            for (int c = 0; c < RC; ++c) zi[c] *= inv;
            for (int m = 0; m < i; ++m) {
                const double l = li[m];
                double* zm = &Z[(size_t)m * RC];
                for (int c = 0; c < RC; ++c) zm[c] -= l * zi[c];
            }
        }
        for (int i = 0; i < p; ++i)
            for (int c = 0; c < nc; ++c) W[(size_t)i * q + c0 + c] = Z[(size_t)i * RC + c];
    });

    // b = mean_y - mean_x W;  W_out output-major [q][p]
    parallel_for(q, n_threads, [&](int j) {
        double s = (double)mean_y[j];
        for (int i = 0; i < p; ++i) s -= (double)mean_x[i] * W[(size_t)i * q + j];
        b_out[j] = (float)s;
        for (int i = 0; i < p; ++i) W_out[(size_t)j * P + i] = (float)W[(size_t)i * q + j];
    });
    return 0;
}

}  // namespace kvmap
