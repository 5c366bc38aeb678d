// Host-side checks of libkvmap built with AddressSanitizer and UndefinedBehaviorSanitizer: the
// C-ABI validation, the host ridge solve (its blocked fp64 Cholesky, register kernel and worker
// pool) and the argument checks of the other entry points, none of which needs a GPU.  Exit
// status 0 when every check holds (the sanitizers abort the run on the first error they find).
#include "../../include/kvmap.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            ++failures;                                    \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
            std::printf(__VA_ARGS__);                      \
            std::printf("\n");                             \
        }                                                  \
    } while (0)

static kvmap_rope rope(double theta, const double* f = nullptr) { return kvmap_rope{theta, 0, KVMAP_ROPE_HALF_SPLIT, f}; }

static void validation() {
    kvmap_dims d{6, 4, 2, 128, 3, 100, KVMAP_DTYPE_BF16};
    const int32_t sel[12] = {0, 2, 5, 1, 3, 4, 5, 4, 3, 0, 1, 2};
    kvmap_rope rs = rope(1e4), rt = rope(5e5);
    CHECK(kvmap_validate_apply(&d, sel, &rs, &rt) == KVMAP_OK, "good call refused: %s", kvmap_last_error());
    int32_t dup[12];
    std::memcpy(dup, sel, sizeof dup);
    dup[4] = dup[3];
    CHECK(kvmap_validate_apply(&d, dup, &rs, &rt) == KVMAP_ERR_SHAPE, "duplicate accepted");
    CHECK(std::strlen(kvmap_last_error()) > 0, "no detail after a refusal");
    dup[4] = 6;
    CHECK(kvmap_validate_apply(&d, dup, &rs, &rt) == KVMAP_ERR_SHAPE, "out of range accepted");
    dup[4] = -1;
    CHECK(kvmap_validate_apply(&d, dup, &rs, &rt) == KVMAP_ERR_SHAPE, "negative accepted");
    CHECK(kvmap_validate_apply(nullptr, sel, &rs, &rt) == KVMAP_ERR_INVALID_ARGUMENT, "NULL dims accepted");
    CHECK(kvmap_validate_apply(&d, nullptr, &rs, &rt) == KVMAP_ERR_INVALID_ARGUMENT, "NULL sel accepted");
    std::vector<double> f(64, 0.5);
    kvmap_rope rf = rope(0.0, f.data());
    CHECK(kvmap_validate_apply(&d, sel, &rf, &rt) == KVMAP_OK, "frequency list refused");
    f[63] = NAN;
    CHECK(kvmap_validate_apply(&d, sel, &rf, &rt) == KVMAP_ERR_INVALID_ARGUMENT, "NaN frequency accepted");
    kvmap_rope ri = rope(1e4);
    ri.style = KVMAP_ROPE_INTERLEAVED;
    CHECK(kvmap_validate_apply(&d, sel, &ri, &rt) == KVMAP_ERR_UNSUPPORTED, "interleaved accepted");
    kvmap_dims big = d;
    big.T = int64_t(1) << 40;
    CHECK(kvmap_validate_apply(&big, sel, &rs, &rt) == KVMAP_ERR_SHAPE, "huge T accepted");
    // buffer addresses (never read): disjoint and aligned, then each refusal
    {
        char* base = reinterpret_cast<char*>(uintptr_t(1) << 40);
        const size_t src = 6 * 2 * 100 * 128 * 2, w = 4 * 256 * 768 * 2, b = 4 * 256 * 2, tgt = 4 * 2 * 100 * 128 * 2;
        const void *sk = base, *sv = base + src, *wk = base + 2 * src, *bk = base + 2 * src + w;
        const void *wv = base + 2 * src + w + 4096, *bv = base + 2 * src + 2 * w + 4096;
        void* tk = base + 2 * src + 2 * w + 8192;
        void* tv = static_cast<char*>(tk) + tgt;
        CHECK(kvmap_validate_apply_buffers(&d, sk, sv, wk, bk, wv, bv, tk, tv) == KVMAP_OK, "good buffers refused: %s",
              kvmap_last_error());
        CHECK(kvmap_validate_apply_buffers(&d, sk, sv, wk, bk, wv, bv, tk, tk) == KVMAP_ERR_INVALID_ARGUMENT,
              "tgt_k == tgt_v accepted");
        CHECK(kvmap_validate_apply_buffers(&d, sk, sv, wk, bk, wv, bv, const_cast<void*>(sv), tv) ==
                  KVMAP_ERR_INVALID_ARGUMENT, "output over an input accepted");
        CHECK(kvmap_validate_apply_buffers(&d, sk, sv, wk, bk, wv, bv, static_cast<char*>(tk) + 8, tv) ==
                  KVMAP_ERR_INVALID_ARGUMENT, "misaligned output accepted");
        CHECK(kvmap_validate_apply_buffers(&d, nullptr, sv, wk, bk, wv, bv, tk, tv) == KVMAP_ERR_INVALID_ARGUMENT,
              "NULL input accepted");
    }
    // statistics call checks on addresses (never read)
    {
        char* base = reinterpret_cast<char*>(uintptr_t(3) << 40);
        kvmap_gram_state gs{};
        gs.p = 520;
        gs.q = 68;
        gs.mean_x = reinterpret_cast<float*>(base);
        gs.mean_y = reinterpret_cast<float*>(base + 4096);
        gs.M_xx = reinterpret_cast<float*>(base + 8192);
        gs.M_xy = reinterpret_cast<float*>(base + 8192 + 520 * 520 * 4);
        const char* xb = base + (size_t(64) << 20);
        const char* yb = xb + (size_t(16) << 20);
        CHECK(kvmap_validate_gram(&gs, xb, yb, 700, KVMAP_DTYPE_BF16) == KVMAP_OK, "good gram call refused: %s",
              kvmap_last_error());
        CHECK(kvmap_validate_gram(&gs, gs.M_xx, yb, 700, KVMAP_DTYPE_BF16) == KVMAP_ERR_INVALID_ARGUMENT,
              "batch over the state accepted");
        CHECK(kvmap_validate_gram(&gs, xb, yb, -1, KVMAP_DTYPE_BF16) == KVMAP_ERR_SHAPE, "negative n_b accepted");
        CHECK(kvmap_validate_gram(nullptr, xb, yb, 700, KVMAP_DTYPE_BF16) == KVMAP_ERR_INVALID_ARGUMENT,
              "NULL state accepted");
    }
    // kvmap_reserve checks the dims before the context
    kvmap_dims zero{};
    CHECK(kvmap_reserve(nullptr, &zero) == KVMAP_ERR_SHAPE, "zero dims reached the workspace arithmetic");
    kvmap_dims d32{1, 1, 1, 32, 1, 16, KVMAP_DTYPE_BF16};
    CHECK(kvmap_reserve(nullptr, &d32) == KVMAP_ERR_UNSUPPORTED, "head dim 32 accepted");
    CHECK(kvmap_reserve(nullptr, &d) == KVMAP_ERR_INVALID_ARGUMENT, "NULL ctx accepted");
    // other entry points refuse NULL contexts / arguments before any device work
    kvmap_gram_state st{};
    CHECK(kvmap_gram(nullptr, nullptr, nullptr, 10, KVMAP_DTYPE_BF16, &st, nullptr) == KVMAP_ERR_INVALID_ARGUMENT, "gram");
    CHECK(kvmap_gram_noalloc(nullptr, nullptr, nullptr, 10, KVMAP_DTYPE_BF16, &st, nullptr) == KVMAP_ERR_INVALID_ARGUMENT,
          "gram_noalloc");
    CHECK(kvmap_gram_merge(nullptr, &st, &st, nullptr) == KVMAP_ERR_INVALID_ARGUMENT, "gram_merge");
    kvmap_fit* fit = nullptr;
    kvmap_fit_config cfg{};
    CHECK(kvmap_fit_create(nullptr, &cfg, &fit) == KVMAP_ERR_INVALID_ARGUMENT && fit == nullptr, "fit_create");
    CHECK(kvmap_fit_destroy(nullptr) == KVMAP_OK, "fit_destroy(NULL)");
    float ms[3];
    CHECK(kvmap_timings(nullptr, 0, ms, 3) == KVMAP_ERR_INVALID_ARGUMENT, "timings");
    CHECK(kvmap_destroy(nullptr) == KVMAP_OK, "destroy(NULL)");
    for (int s = -1; s <= 8; ++s) CHECK(kvmap_status_string(s) != nullptr, "status string %d", s);
    CHECK(kvmap_version() == KVMAP_VERSION, "version");
    // a context on a machine with no GPU reports a device error; with one, it is created and freed
    kvmap_ctx* c = nullptr;
    const int st_create = kvmap_create(&c, 0);
    CHECK((st_create == KVMAP_OK) == (c != nullptr), "create status %d vs handle", st_create);
    if (c) kvmap_destroy(c);
}

// W = (sym(M) + lambda I)^-1 M_xy with b = mean_y - mean_x W: checked by its residual
static void ridge_case(int p, int q, int threads, std::mt19937_64& g) {
    const int n = p + 9;
    std::normal_distribution<double> nd;
    std::vector<double> X((size_t)n * p), Y((size_t)n * q);
    for (auto& v : X) v = nd(g);
    for (auto& v : Y) v = nd(g);
    std::vector<float> Mxx((size_t)p * p), Mxy((size_t)p * q), mx(p), my(q);
    for (int i = 0; i < p; ++i) {
        mx[i] = (float)nd(g);
        for (int j = 0; j < p; ++j) {
            double s = 0;
            for (int r = 0; r < n; ++r) s += X[(size_t)r * p + i] * X[(size_t)r * p + j];
            Mxx[(size_t)i * p + j] = (float)s;
        }
        for (int j = 0; j < q; ++j) {
            double s = 0;
            for (int r = 0; r < n; ++r) s += X[(size_t)r * p + i] * Y[(size_t)r * q + j];
            Mxy[(size_t)i * q + j] = (float)s;
        }
    }
    for (auto& v : my) v = (float)nd(g);
    const double lam = 0.01;
    std::vector<float> W((size_t)q * p, NAN), b(q, NAN);
    const int st = kvmap_ridge_solve_host(p, q, mx.data(), my.data(), Mxx.data(), Mxy.data(), lam, W.data(), b.data(), threads);
    CHECK(st == KVMAP_OK, "p=%d q=%d threads=%d: status %d (%s)", p, q, threads, st, kvmap_last_error());
    if (st) return;
    double worst = 0, worst_b = 0;
    for (int c = 0; c < q; ++c) {
        double wn = 0, bn = std::fabs(my[c]);
        for (int i = 0; i < p; ++i) wn = std::fmax(wn, std::fabs(W[(size_t)c * p + i]));
        for (int i = 0; i < p; ++i) {  // row i of (upper-triangle symmetric M + lambda I) w_c - M_xy[i][c]
            double s = lam * W[(size_t)c * p + i];
            for (int j = 0; j < p; ++j) {
                const float m = i <= j ? Mxx[(size_t)i * p + j] : Mxx[(size_t)j * p + i];
                s += (double)m * W[(size_t)c * p + j];
            }
            worst = std::fmax(worst, std::fabs(s - Mxy[(size_t)i * q + c]) / (1.0 + (double)n * wn));
        }
        double bb = my[c];
        for (int i = 0; i < p; ++i) bb -= (double)mx[i] * W[(size_t)c * p + i];
        worst_b = std::fmax(worst_b, std::fabs(bb - b[c]) / (1.0 + bn + wn * p));
    }
    CHECK(worst < 1e-5 && worst_b < 1e-6, "p=%d q=%d threads=%d: residual %.3g, intercept %.3g", p, q, threads, worst,
          worst_b);
}

static void ridge() {
    std::mt19937_64 g(2026);
    const int ps[] = {1, 7, 64, 65, 130, 257};
    const int qs[] = {1, 5, 70};
    const int ths[] = {1, 3, 0};
    for (int p : ps)
        for (int q : qs)
            for (int t : ths) ridge_case(p, q, t, g);
    // not positive definite: M = -I
    const int p = 9, q = 2;
    std::vector<float> M((size_t)p * p, 0.f), Mxy((size_t)p * q, 1.f), mx(p, 0.f), my(q, 0.f), W((size_t)p * q), b(q);
    for (int i = 0; i < p; ++i) M[(size_t)i * p + i] = -1.f;
    CHECK(kvmap_ridge_solve_host(p, q, mx.data(), my.data(), M.data(), Mxy.data(), 0.01, W.data(), b.data(), 2) ==
              KVMAP_ERR_NOT_SPD, "negative definite system solved");
    CHECK(kvmap_ridge_solve_host(p, q, mx.data(), my.data(), M.data(), Mxy.data(), -1.0, W.data(), b.data(), 2) ==
              KVMAP_ERR_INVALID_ARGUMENT, "negative lambda accepted");
    CHECK(kvmap_ridge_solve_host(p, q, nullptr, my.data(), M.data(), Mxy.data(), 0.01, W.data(), b.data(), 2) ==
              KVMAP_ERR_INVALID_ARGUMENT, "NULL accepted");
    CHECK(kvmap_ridge_solve_host(0, q, mx.data(), my.data(), M.data(), Mxy.data(), 0.01, W.data(), b.data(), 2) ==
              KVMAP_ERR_SHAPE, "p = 0 accepted");
}

int main() {
    validation();
    ridge();
    std::printf("host checks: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}
