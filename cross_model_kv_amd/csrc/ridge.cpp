// Closed-form ridge on the host in float64 (KVBridge README, fitting section headed
// "Loading": W = (X^T X + lambda I)^-1 X^T Y, b = Ybar - Xbar W; reactapp.top article, section
// "Eine lineare Bruecke reicht": lambda = 0.01 added to the centred Gram, intercept from the
// means, so the intercept is not penalised).
//
//   A = sym(M_xx) + lambda I = L L^T          blocked right-looking Cholesky
//   L Z = M_xy,  L^T W = Z                    blocked forward / back substitution
//   b = mean_y - mean_x W
//
// Every O(p^3) and O(p^2 q) part is a product C -= A B done by one register-blocked kernel
// (6 x 8 doubles of C in 12 AVX2 registers; per k a broadcast of A's 6 values and two vector
// loads of B) on operands packed into the kernel's order, over tiles handed to the threads of
// a pool started once per solve:
//   * the trailing update of each Cholesky panel, A22 -= P P^T (lower triangle only);
//   * the substitutions' updates, Z_i -= L_ik Z_k below each diagonal block and
//     W_i -= L_ki^T W_k above it.
// The diagonal blocks themselves (a b x b factor, the panel's b x b triangular solve and the
// b x b substitutions over all q columns) are the only unblocked parts: O(p b (b + q)) of the
// O(p^3 / 3 + 2 p^2 q) work.

#include "ridge.h"

#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <cmath>
#include <cstdint>
#include <functional>
#include <memory>
#include <mutex>
#include <system_error>
#include <thread>
#include <vector>

namespace kvmap {

namespace {

// Workers started once per solve; each run() hands items 0..n-1 out through an atomic
// counter to the workers and the calling thread and returns when all of them are done.
// (Starting threads per parallel step cost more than the small steps themselves.)
class Pool {
  public:
    explicit Pool(int n_threads) {
        for (int t = 1; t < n_threads; ++t) {
            try {
                workers_.emplace_back([this] { loop(); });
            } catch (const std::system_error&) {
                break;  // the system refused another thread: run on those that did start
            }
        }
        n_ = (int)workers_.size() + 1;
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
            ++gen_;
        }
        start_.notify_all();
        for (auto& w : workers_) w.join();
    }
    template <typename Fn>
    void run(int n_items, Fn&& fn) {
        if (n_items <= 0) return;
        if (n_ == 1 || n_items == 1) {
            for (int i = 0; i < n_items; ++i) fn(i);
            return;
        }
        std::function<void(int)> job(std::forward<Fn>(fn));
        {
            std::lock_guard<std::mutex> lk(mu_);
            job_ = &job;
            items_ = n_items;
            next_.store(0);
            pending_ = n_ - 1;
            ++gen_;
        }
        start_.notify_all();
        work();
        std::unique_lock<std::mutex> lk(mu_);
        done_.wait(lk, [this] { return pending_ == 0; });
        job_ = nullptr;
    }

  private:
    void work() {
        for (int i = next_.fetch_add(1); i < items_; i = next_.fetch_add(1)) (*job_)(i);
    }
    void loop() {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(mu_);
        for (;;) {
            start_.wait(lk, [&] { return gen_ != seen; });
            seen = gen_;
            if (stop_) return;
            lk.unlock();
            work();
            lk.lock();
            if (--pending_ == 0) done_.notify_one();
        }
    }
    int n_ = 1;
    std::vector<std::thread> workers_;
    std::mutex mu_;
    std::condition_variable start_, done_;
    std::function<void(int)>* job_ = nullptr;
    int items_ = 0;
    std::atomic<int> next_{0};
    int pending_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

constexpr int NB = 128;  // panel / diagonal block width
constexpr int MR = 6;    // rows of C held in registers
constexpr int NR = 8;    // columns of C held in registers (two 4-double vectors)
constexpr int MC = 16;   // register blocks of rows per task (96 rows)
constexpr int NC = 16;   // register blocks of columns per task (128 columns)
constexpr int TT = 64;   // rows or columns per task of the input and output transposes

// Operands of C -= A B packed into the register kernel's order, so that its loads are
// contiguous whatever the source strides: A [m][k] as MR-row slivers [ceil(m/MR)][k][MR],
// B [k][n] as NR-column slivers [ceil(n/NR)][k][NR]; rows or columns beyond m or n are zero.
// A given row-major [m][k] (lda), or, with `trans`, given as its transpose [k][m] (lda).
void pack_a(int m, int k, const double* A, size_t lda, bool trans, std::vector<double>& out, Pool& pool) {
    const int ms = (m + MR - 1) / MR;
    out.assign((size_t)ms * k * MR, 0.0);
    pool.run(ms, [&](int s) {
        double* o = out.data() + (size_t)s * k * MR;
        const int nr = std::min(MR, m - s * MR);
        if (trans) {
            for (int t = 0; t < k; ++t) {
                const double* a = A + (size_t)t * lda + s * MR;
                for (int r = 0; r < nr; ++r) o[(size_t)t * MR + r] = a[r];
            }
        } else {
            for (int r = 0; r < nr; ++r) {
                const double* a = A + (size_t)(s * MR + r) * lda;
                for (int t = 0; t < k; ++t) o[(size_t)t * MR + r] = a[t];
            }
        }
    });
}

// B given row-major [k][n] (ldb), or, with `trans`, given as its transpose [n][k] (ldb).
void pack_b(int k, int n, const double* B, size_t ldb, bool trans, std::vector<double>& out, Pool& pool) {
    const int ns = (n + NR - 1) / NR;
    out.assign((size_t)ns * k * NR, 0.0);
    pool.run(ns, [&](int s) {
        double* o = out.data() + (size_t)s * k * NR;
        const int nc = std::min(NR, n - s * NR);
        if (trans) {
            for (int c = 0; c < nc; ++c) {
                const double* b = B + (size_t)(s * NR + c) * ldb;
                for (int t = 0; t < k; ++t) o[(size_t)t * NR + c] = b[t];
            }
        } else {
            for (int t = 0; t < k; ++t) {
                const double* b = B + (size_t)t * ldb + s * NR;
                for (int c = 0; c < nc; ++c) o[(size_t)t * NR + c] = b[c];
            }
        }
    });
}

// acc[MR x NR] = a-sliver^T b-sliver over k: a[t][MR], b[t][NR] contiguous.
inline void kernel_6x8(int k, const double* a, const double* b, __m256d c[MR][2]) {
    for (int r = 0; r < MR; ++r) c[r][0] = c[r][1] = _mm256_setzero_pd();
    for (int t = 0; t < k; ++t, a += MR, b += NR) {
        const __m256d b0 = _mm256_loadu_pd(b);
        const __m256d b1 = _mm256_loadu_pd(b + 4);
        for (int r = 0; r < MR; ++r) {
            const __m256d x = _mm256_broadcast_sd(a + r);
            c[r][0] = _mm256_fmadd_pd(x, b0, c[r][0]);
            c[r][1] = _mm256_fmadd_pd(x, b1, c[r][1]);
        }
    }
}

// C[m x n] -= A B from packed operands (pack_a, pack_b with the same m, n, k), over tasks of
// MC x NC register blocks in parallel.  `lower` skips register blocks lying wholly above the
// diagonal (the trailing update: only the lower triangle of C is ever read).
void gemm_sub(int m, int n, int k, const std::vector<double>& Ap, const std::vector<double>& Bp, double* C,
              size_t ldc, bool lower, Pool& pool) {
    const int ms = (m + MR - 1) / MR, ns = (n + NR - 1) / NR;
    const int tm = (ms + MC - 1) / MC, tn = (ns + NC - 1) / NC;
    std::vector<std::pair<int, int>> tasks;
    tasks.reserve((size_t)tm * tn);
    for (int i = 0; i < tm; ++i)
        for (int j = 0; j < tn; ++j)
            if (!lower || j * NC * NR <= std::min(m, (i + 1) * MC * MR) - 1) tasks.emplace_back(i, j);
    pool.run((int)tasks.size(), [&](int u) {
        const int si1 = std::min(ms, (tasks[u].first + 1) * MC);
        const int sj1 = std::min(ns, (tasks[u].second + 1) * NC);
        for (int sj = tasks[u].second * NC; sj < sj1; ++sj) {
            const double* b = Bp.data() + (size_t)sj * k * NR;
            const int j0 = sj * NR, nc = std::min(NR, n - j0);
            for (int si = tasks[u].first * MC; si < si1; ++si) {
                const int i0 = si * MR, nr = std::min(MR, m - i0);
                if (lower && j0 > i0 + nr - 1) continue;
                __m256d c[MR][2];
                kernel_6x8(k, Ap.data() + (size_t)si * k * MR, b, c);
                if (nr == MR && nc == NR) {
                    for (int r = 0; r < MR; ++r) {
                        double* cr = C + (size_t)(i0 + r) * ldc + j0;
                        _mm256_storeu_pd(cr, _mm256_sub_pd(_mm256_loadu_pd(cr), c[r][0]));
                        _mm256_storeu_pd(cr + 4, _mm256_sub_pd(_mm256_loadu_pd(cr + 4), c[r][1]));
                    }
                } else {
                    alignas(32) double t[MR][NR];
                    for (int r = 0; r < MR; ++r) {
                        _mm256_store_pd(&t[r][0], c[r][0]);
                        _mm256_store_pd(&t[r][4], c[r][1]);
                    }
                    for (int r = 0; r < nr; ++r)
                        for (int cc = 0; cc < nc; ++cc) C[(size_t)(i0 + r) * ldc + j0 + cc] -= t[r][cc];
                }
            }
        }
    });
}

}  // namespace

int ridge_solve_f64(int p, int q, const float* mean_x, const float* mean_y, const float* M_xx,
                    const float* M_xy, double lambda, float* W_out, float* b_out,
                    int n_threads) {
    if (n_threads <= 0) n_threads = (int)std::max(1u, std::thread::hardware_concurrency());
    n_threads = std::min(n_threads, (p + TT - 1) / TT);  // small systems: starting threads dominates
    const size_t P = (size_t)p;
    Pool pool(n_threads);
    // Lower triangle of A from the upper triangle of M_xx, plus lambda on the diagonal, the upper
    // triangle zero; by blocks of TT rows, so that M_xx is read a row segment at a time.
    std::unique_ptr<double[]> A_buf(new double[P * P]);
    double* A = A_buf.get();
    pool.run((p + TT - 1) / TT, [&](int bi) {
        const int i0 = bi * TT, i1 = std::min(p, i0 + TT);
        for (int i = i0; i < i1; ++i) std::fill(A + (size_t)i * P + i + 1, A + (size_t)(i + 1) * P, 0.0);
        for (int j = 0; j < i1; ++j) {
            const float* src = M_xx + (size_t)j * P;
            for (int i = std::max(i0, j); i < i1; ++i) A[(size_t)i * P + j] = (double)src[i];
        }
        for (int i = i0; i < i1; ++i) A[(size_t)i * P + i] += lambda;
    });

    // ---- A = L L^T ----
    std::vector<double> Ap, Bp;  // packed operands of the current product
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
        // 2. panel rows below: row_i <- row_i L_kk^-T
        pool.run((nr + 63) / 64, [&](int blk) {
            for (int i = r0 + blk * 64; i < std::min(p, r0 + blk * 64 + 64); ++i) {
                double* row = &A[(size_t)i * P + k];
                for (int j = 0; j < b; ++j) {
                    double t = row[j];
                    const double* lj = &A[(size_t)(k + j) * P + k];
                    for (int m = 0; m < j; ++m) t -= row[m] * lj[m];
                    row[j] = t / lj[j];
                }
            }
        });
        // 3. trailing update of the lower triangle: A22 -= P P^T, P the panel just solved
        const double* pan = &A[(size_t)r0 * P + k];
        pack_a(nr, b, pan, P, false, Ap, pool);
        pack_b(b, nr, pan, P, true, Bp, pool);
        gemm_sub(nr, nr, b, Ap, Bp, &A[(size_t)r0 * P + r0], P, true, pool);
    }

    // ---- L Z = M_xy, then L^T W = Z, in place in W [p][q] ----
    std::unique_ptr<double[]> W_buf(new double[P * (size_t)q]);
    double* W = W_buf.get();
    pool.run(p, [&](int i) {
        for (int c = 0; c < q; ++c) W[(size_t)i * q + c] = (double)M_xy[(size_t)i * q + c];
    });
    const int cq = 64;  // right-hand-side columns per task of a diagonal-block solve
    const int ncq = (q + cq - 1) / cq;
    for (int k = 0; k < p; k += NB) {
        const int b = std::min(NB, p - k);
        // Z_k = L_kk^-1 Z_k
        pool.run(ncq, [&](int ch) {
            const int c0 = ch * cq, c1 = std::min(q, c0 + cq);
            for (int i = k; i < k + b; ++i) {
                double* zi = &W[(size_t)i * q];
                const double* li = &A[(size_t)i * P];
                for (int m = k; m < i; ++m) {
                    const double l = li[m];
                    const double* zm = &W[(size_t)m * q];
                    for (int c = c0; c < c1; ++c) zi[c] -= l * zm[c];
                }
                const double inv = 1.0 / li[i];
                for (int c = c0; c < c1; ++c) zi[c] *= inv;
            }
        });
        // Z_i -= L_ik Z_k for the rows below
        const int r0 = k + b;
        if (r0 < p) {
            pack_a(p - r0, b, &A[(size_t)r0 * P + k], P, false, Ap, pool);
            pack_b(b, q, &W[(size_t)k * q], (size_t)q, false, Bp, pool);
            gemm_sub(p - r0, q, b, Ap, Bp, &W[(size_t)r0 * q], (size_t)q, false, pool);
        }
    }
    const int last = (p - 1) / NB * NB;
    for (int k = last; k >= 0; k -= NB) {
        const int b = std::min(NB, p - k);
        // W_k = L_kk^-T W_k
        pool.run(ncq, [&](int ch) {
            const int c0 = ch * cq, c1 = std::min(q, c0 + cq);
            for (int i = k + b - 1; i >= k; --i) {
                double* wi = &W[(size_t)i * q];
                const double inv = 1.0 / A[(size_t)i * P + i];
                for (int c = c0; c < c1; ++c) wi[c] *= inv;
                for (int m = k; m < i; ++m) {
                    const double l = A[(size_t)i * P + m];
                    double* wm = &W[(size_t)m * q];
                    for (int c = c0; c < c1; ++c) wm[c] -= l * wi[c];
                }
            }
        });
        // W_i -= L_ki^T W_k for the rows above: the A operand is block row k of L, transposed
        if (k > 0) {
            pack_a(k, b, &A[(size_t)k * P], P, true, Ap, pool);
            pack_b(b, q, &W[(size_t)k * q], (size_t)q, false, Bp, pool);
            gemm_sub(k, q, b, Ap, Bp, W, (size_t)q, false, pool);
        }
    }

    // b = mean_y - mean_x W and W_out = W^T (output-major [q][p]), by blocks of TT columns of W
    pool.run((q + TT - 1) / TT, [&](int bj) {
        const int j0 = bj * TT, j1 = std::min(q, j0 + TT);
        double acc[TT];
        for (int j = j0; j < j1; ++j) acc[j - j0] = (double)mean_y[j];
        for (int i = 0; i < p; ++i) {
            const double* wi = W + (size_t)i * q;
            const double mx = (double)mean_x[i];
            for (int j = j0; j < j1; ++j) {
                acc[j - j0] -= mx * wi[j];
                W_out[(size_t)j * P + i] = (float)wi[j];
            }
        }
        for (int j = j0; j < j1; ++j) b_out[j] = (float)acc[j - j0];
    });
    return 0;
}

}  // namespace kvmap
