// End-to-end fit driver over the C-ABI (KVBridge README, fitting section headed "Loading":
// a two-stage, multi-pass fit over re-iterable calibration data that keeps only centered
// statistics, with target-layer blocks bounding memory; "What ships": source layers scored one
// at a time by R^2 averaged over target heads, the best k per target layer kept, then
// one ridge map per target layer for keys and one for values).
//
// The driver owns the statistics of one stage at a time and calls the library's own entry
// points for every step: kvmap_cache_rows (gather + strip RoPE into token rows), kvmap_gram
// (Chan-merged centered statistics), kvmap_ridge_r2_batch (stage-1 scores per target head) and
// kvmap_ridge_solve_device_batch (stage-2 maps).  The selection itself (average over heads and
// {K, V}, top-k) is the one kernel of this file.
//
// Stage 1 feeds a group of source layers (as many as fit 65,536 features) as ONE Gram state per
// K/V against the rows of a block of target layers: every layer's co-moments come out of one
// launch per batch, the target rows are split once per batch rather than once per source
// layer, and the launch has enough tiles to fill the chip.
//
// One pass, when every source layer fits one state and every target layer one block (the
// 14B->32B shape: 40 x 1024 source features, 64 x 1024 target features): the state keeps the
// FULL source Gram (all pairs of source layers; 6.7 GB per K/V at that shape, which HBM holds).
// Every statistic a map needs is then a block of it: target t's M_xx is the blocks of its
// selected layers, its M_xy the rows of those layers and the columns of t.  Selection and all
// maps come from this one pass over the calibration data -- no second pass, and fewer co-moment
// FLOPs than per-target states, since target layers that share source layers share blocks.
// Otherwise M_xx is kept block-diagonal (one block per source layer) for the selection and a
// second stage of passes accumulates per-target statistics.

#include "../../include/kvmap.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "common.h"
#include "internal.h"

using namespace kvmap;

namespace kvmap {

namespace {

constexpr int kMaxFitSrcLayers = 1024;
constexpr int kMaxGramWidth = 65536;

// a ranks above b: larger score, then lower index; NaN scores rank below every number
__device__ __forceinline__ bool ranks_above(double a, int ia, double b, int ib) {
    const bool na = a != a, nb = b != b;
    if (na != nb) return nb;
    if (!na && a != b) return a > b;
    return ia < ib;
}

// One workgroup per target layer; lane 0 selects (L_src <= 1024, k <= L_src).
__global__ __launch_bounds__(64) void fit_select_kernel(const double* __restrict__ r2, int L_src, int L_tgt,
                                                        int H, int k, double* __restrict__ scores,
                                                        int32_t* __restrict__ sel) {
    __shared__ double sc[kMaxFitSrcLayers];
    __shared__ unsigned char taken[kMaxFitSrcLayers];
    const int t = blockIdx.x;
    for (int s = threadIdx.x; s < L_src; s += 64) {
        double acc = 0.0;
        for (int kv = 0; kv < 2; ++kv)
            for (int h = 0; h < H; ++h) acc += r2[(((size_t)kv * L_src + s) * L_tgt + t) * H + h];
        const double v = acc / (2.0 * H);
        sc[s] = v;
        taken[s] = 0;
        scores[(size_t)t * L_src + s] = v;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int s = 0; s < L_src; ++s)
            if (!taken[s] && (best < 0 || ranks_above(sc[s], s, sc[best], best))) best = s;
        taken[best] = 1;
    }
    int o = 0;
    for (int s = 0; s < L_src; ++s)
        if (taken[s]) sel[(size_t)t * k + o++] = s;
}

}  // namespace

hipError_t launch_fit_select(const double* r2, int L_src, int L_tgt, int H, int k, double* scores, int32_t* sel,
                             hipStream_t s) {
    hipLaunchKernelGGL(fit_select_kernel, dim3(L_tgt), dim3(64), 0, s, r2, L_src, L_tgt, H, k, scores, sel);
    return hipGetLastError();
}

}  // namespace kvmap

// ---------------------------------------------------------------------------------------
// the driver
// ---------------------------------------------------------------------------------------

struct kvmap_fit {
    kvmap_ctx* ctx = nullptr;
    kvmap_fit_config cfg{};
    int device = 0;
    int N = 0, F = 0;                  // H*d, k*H*d
    int sel_block = 0, map_block = 0;  // target layers per pass of each stage
    int group = 0, groups = 0;         // stage 1: source layers per Gram state, states per K/V
    bool one_pass = false;             // full source Gram in stage 1, maps gathered from it
    float* gbuf = nullptr;             // one-pass mode: gathered blocks (diagonal blocks, then maps)
    size_t gbuf_floats = 0;
    int sel_passes = 0, map_passes = 0;
    int pass = -1;                     // index of the open pass, -1 before the first
    int stage = 0, t0 = 0, t1 = 0;
    int64_t n_pass = 0, n_first = -1;  // tokens fed to the open pass / to the first pass
    std::vector<int32_t> sel;          // host copy of layer_sel [L_tgt][k]
    std::vector<double> freq_src, freq_tgt;  // the models' own rotary frequencies, if given
    std::vector<kvmap_gram_state> states;
    float* state_mem = nullptr;
    double* r2 = nullptr;              // [2][L_src][L_tgt][H]
    double* own_scores = nullptr;      // when cfg.scores is NULL
    void* xrows = nullptr;
    void* yrows = nullptr;
    size_t xcap = 0, ycap = 0;
    // Stage 1 with one source group: the rows of consecutive sequences are gathered per K/V
    // into these buffers and merged together, up to kAccRows rows per kvmap_gram call.
    void* accx[2] = {nullptr, nullptr};
    void* accy[2] = {nullptr, nullptr};
    size_t accx_cap = 0, accy_cap = 0;
    int64_t n_acc = 0;
};

namespace {

#define FIT_HIP(call)                                                                                 \
    do {                                                                                              \
        hipError_t e_ = (call);                                                                       \
        if (e_ != hipSuccess)                                                                         \
            return report(e_ == hipErrorOutOfMemory ? KVMAP_ERR_OUT_OF_MEMORY : KVMAP_ERR_DEVICE,     \
                          "%s: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__);         \
    } while (0)

#define FIT_TRY(call)             \
    do {                          \
        const int r_ = (call);    \
        if (r_ != KVMAP_OK) return r_; \
    } while (0)

struct FitDevice {
    int prev = -1;
    explicit FitDevice(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        (void)hipSetDevice(dev);
    }
    ~FitDevice() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

size_t esize(int32_t dtype) { return dtype == KVMAP_DTYPE_BF16 ? 2 : 4; }

void free_stage(kvmap_fit* f) {
    if (f->state_mem) {
        (void)hipDeviceSynchronize();
        (void)hipFree(f->state_mem);
    }
    f->state_mem = nullptr;
    f->states.clear();
}

// Lay out n states of (p, q) in one allocation; every array starts 16-byte aligned since p, q
// are multiples of 64.
// Lay out states of widths ps[i] (all of one q) in one allocation; every array starts 16-byte
// aligned since p, q and the block are multiples of 64.  xx_block > 0: M_xx block-diagonal.
int alloc_states(kvmap_fit* f, const std::vector<int>& ps, int q, bool keep_ss_y, int xx_block) {
    free_stage(f);
    size_t total = 0;
    for (int p : ps)
        total += (size_t)p + q + (size_t)p * (xx_block ? xx_block : p) + (size_t)p * q + (keep_ss_y ? q : 0);
    FIT_HIP(hipMalloc((void**)&f->state_mem, total * sizeof(float)));
    f->states.assign(ps.size(), kvmap_gram_state{});
    float* b = f->state_mem;
    for (size_t i = 0; i < ps.size(); ++i) {
        const int p = ps[i];
        kvmap_gram_state& st = f->states[i];
        st.n = 0;
        st.p = p;
        st.q = q;
        st.xx_block = xx_block;
        st.mean_x = b; b += p;
        st.mean_y = b; b += q;
        st.M_xx = b; b += (size_t)p * (xx_block ? xx_block : p);
        st.M_xy = b; b += (size_t)p * q;
        st.ss_y = keep_ss_y ? b : nullptr;
        b += keep_ss_y ? q : 0;
    }
    return KVMAP_OK;
}

// Blocks of a gathered matrix: block i of the output is block b[i] of the input.
struct BlockList {
    int n;
    int b[kMaxRowLayers];
};

// out[(bi NR + r) ldo + bj NC + c] = in[(rows.b[bi] NR + r) ldi + cols.b[bj] NC + c]; NC and the
// leading dimensions are multiples of 4 (float4 copies).
__global__ __launch_bounds__(256) void gather_blocks_kernel(float* __restrict__ out, int64_t ldo,
                                                            const float* __restrict__ in, int64_t ldi,
                                                            const BlockList rows, const BlockList cols, int NR,
                                                            int NC) {
    const int64_t nrow = (int64_t)rows.n * NR;
    const int64_t row4 = (int64_t)cols.n * NC / 4;
    const int64_t total = nrow * row4;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t R = idx / row4;
        const int C = (int)(idx - R * row4) * 4;
        const int bi = (int)(R / NR), r = (int)(R - (int64_t)bi * NR);
        const int bj = C / NC, c = C - bj * NC;
        const float4 v = *(const float4*)(in + ((int64_t)rows.b[bi] * NR + r) * ldi + (int64_t)cols.b[bj] * NC + c);
        *(float4*)(out + R * ldo + C) = v;
    }
}

hipError_t gather_blocks(float* out, int64_t ldo, const float* in, int64_t ldi, const BlockList& rows,
                         const BlockList& cols, int NR, int NC, hipStream_t s) {
    const int64_t total = (int64_t)rows.n * NR * cols.n * NC / 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 16384);
    hipLaunchKernelGGL(gather_blocks_kernel, dim3(std::max(1u, blocks)), dim3(256), 0, s, out, ldo, in, ldi, rows,
                       cols, NR, NC);
    return hipGetLastError();
}

BlockList one_block(int b) {
    BlockList l{};
    l.n = 1;
    l.b[0] = b;
    return l;
}

int ensure_gbuf(kvmap_fit* f, size_t floats, hipStream_t s) {
    if (floats <= f->gbuf_floats) return KVMAP_OK;
    FIT_HIP(hipStreamSynchronize(s));
    (void)hipFree(f->gbuf);
    f->gbuf = nullptr;
    f->gbuf_floats = 0;
    FIT_HIP(hipMalloc((void**)&f->gbuf, floats * sizeof(float)));
    f->gbuf_floats = floats;
    return KVMAP_OK;
}

// One-pass mode, after the selection: the maps of all target layers from the stage-1 states
// (state kv: p = L_src N, full M_xx, q = L_tgt N), gathered a few systems at a time into
// per-target states and solved in batches.
int solve_maps_from_full(kvmap_fit* f, hipStream_t s) {
    const kvmap_fit_config& c = f->cfg;
    const int N = f->N, F = f->F, k = c.k;
    const size_t per = (size_t)F * F + (size_t)F * N + F;  // M_xx, M_xy, mean_x of one system
    const int chunk_t = 8;                                  // target layers (x K, V) per batch
    FIT_TRY(ensure_gbuf(f, per * 2 * chunk_t, s));
    const size_t es = esize(c.out_dtype);
    for (int t0 = 0; t0 < c.L_tgt; t0 += chunk_t) {
        const int t1 = std::min(c.L_tgt, t0 + chunk_t);
        std::vector<kvmap_gram_state> sys;
        std::vector<void*> Ws, bs;
        float* g = f->gbuf;
        for (int t = t0; t < t1; ++t) {
            BlockList sel{};
            sel.n = k;
            for (int j = 0; j < k; ++j) sel.b[j] = f->sel[(size_t)t * k + j];
            for (int kv = 0; kv < 2; ++kv) {
                const kvmap_gram_state& G = f->states[kv];
                kvmap_gram_state v{};
                v.n = G.n;
                v.p = F;
                v.q = N;
                v.M_xx = g; g += (size_t)F * F;
                v.M_xy = g; g += (size_t)F * N;
                v.mean_x = g; g += F;
                v.mean_y = G.mean_y + (size_t)t * N;
                FIT_HIP(gather_blocks(v.M_xx, F, G.M_xx, G.p, sel, sel, N, N, s));
                FIT_HIP(gather_blocks(v.M_xy, N, G.M_xy, G.q, sel, one_block(t), N, N, s));
                FIT_HIP(gather_blocks(v.mean_x, F, G.mean_x, 0, one_block(0), sel, 1, N, s));
                sys.push_back(v);
                Ws.push_back((char*)(kv ? c.W_v : c.W_k) + (size_t)t * N * F * es);
                bs.push_back((char*)(kv ? c.b_v : c.b_k) + (size_t)t * N * es);
            }
        }
        std::vector<const kvmap_gram_state*> st;
        for (const auto& v : sys) st.push_back(&v);
        FIT_TRY(kvmap_ridge_solve_device_batch(f->ctx, st.data(), (int)st.size(), c.lambda, Ws.data(), bs.data(),
                                               c.out_dtype, s));
    }
    return KVMAP_OK;
}

// Rows per accumulated stage-1 batch (the statistics' sub-batch size): short calibration
// sequences are merged in batches of this many rows, so each co-moment launch has a long
// reduction and the per-launch costs (column sums, split, epilogue merge) are shared.
constexpr int64_t kAccRows = 16384;

// Merge the accumulated stage-1 rows into the states (one source group).
int flush_rows(kvmap_fit* f, hipStream_t s) {
    if (f->n_acc == 0) return KVMAP_OK;
    for (int kv = 0; kv < 2; ++kv)
        FIT_TRY(kvmap_gram(f->ctx, f->accx[kv], f->accy[kv], f->n_acc, f->cfg.dtype, &f->states[kv], s));
    f->n_acc = 0;
    return KVMAP_OK;
}

// Source layers of stage-1 group g: [g * group, min(L_src, (g + 1) * group))
int group_layers(const kvmap_fit* f, int g) { return std::min(f->cfg.L_src, (g + 1) * f->group) - g * f->group; }

int ensure_rows(void** buf, size_t* cap, size_t need, hipStream_t s) {
    if (need <= *cap) return KVMAP_OK;
    FIT_HIP(hipStreamSynchronize(s));
    (void)hipFree(*buf);
    *buf = nullptr;
    *cap = 0;
    FIT_HIP(hipMalloc(buf, need));
    *cap = need;
    return KVMAP_OK;
}

// Open pass number f->pass (0-based over both stages): block bounds, states sized and reset.
int open_pass(kvmap_fit* f, hipStream_t s) {
    const kvmap_fit_config& c = f->cfg;
    f->n_pass = 0;
    if (f->pass < f->sel_passes) {
        f->stage = 1;
        f->t0 = f->pass * f->sel_block;
        f->t1 = std::min(c.L_tgt, f->t0 + f->sel_block);
        if (f->pass == 0) {
            std::vector<int> ps;
            for (int kv = 0; kv < 2; ++kv)
                for (int g = 0; g < f->groups; ++g) ps.push_back(group_layers(f, g) * f->N);
            FIT_TRY(alloc_states(f, ps, f->sel_block * f->N, true, f->one_pass ? 0 : f->N));
        }
        for (auto& st : f->states) {
            st.q = (f->t1 - f->t0) * f->N;
            FIT_TRY(kvmap_gram_reset(f->ctx, &st, s));
        }
        return KVMAP_OK;
    }
    const int b = f->pass - f->sel_passes;
    f->stage = 2;
    f->t0 = b * f->map_block;
    f->t1 = std::min(c.L_tgt, f->t0 + f->map_block);
    if (b == 0) FIT_TRY(alloc_states(f, std::vector<int>(2 * f->map_block, f->F), f->N, false, 0));
    for (int i = 0; i < 2 * (f->t1 - f->t0); ++i) FIT_TRY(kvmap_gram_reset(f->ctx, &f->states[i], s));
    return KVMAP_OK;
}

// Close the open pass: stage 1 scores its block (and the last one selects); stage 2 solves.
int close_pass(kvmap_fit* f, hipStream_t s) {
    const kvmap_fit_config& c = f->cfg;
    if (f->n_pass == 0) return report(KVMAP_ERR_SHAPE, "kvmap_fit_next_pass: pass %d saw no tokens", f->pass);
    if (f->n_first >= 0 && f->n_pass != f->n_first)
        return report(KVMAP_ERR_SHAPE, "kvmap_fit_next_pass: pass %d saw %lld tokens, the first pass %lld", f->pass,
                      (long long)f->n_pass, (long long)f->n_first);
    if (f->n_first < 0) f->n_first = f->n_pass;
    if (f->stage == 1) {
        FIT_TRY(flush_rows(f, s));
        const int H = c.H_kv;
        // one view per (K/V, source layer): the layer's diagonal block of its group's state (in
        // one-pass mode copied out of the full M_xx, which the views cannot address)
        const int N = f->N;
        if (f->one_pass) {
            FIT_TRY(ensure_gbuf(f, (size_t)2 * c.L_src * N * N, s));
            for (int kv = 0; kv < 2; ++kv)
                for (int sl = 0; sl < c.L_src; ++sl)
                    FIT_HIP(gather_blocks(f->gbuf + ((size_t)kv * c.L_src + sl) * N * N, N, f->states[kv].M_xx,
                                          f->states[kv].p, one_block(sl), one_block(sl), N, N, s));
        }
        std::vector<kvmap_gram_state> views;
        std::vector<double*> out;
        for (int kv = 0; kv < 2; ++kv)
            for (int sl = 0; sl < c.L_src; ++sl) {
                const kvmap_gram_state& G = f->states[kv * f->groups + sl / f->group];
                const int j = sl % f->group;
                kvmap_gram_state v = G;
                v.p = N;
                v.xx_block = 0;
                v.mean_x = G.mean_x + (size_t)j * N;
                v.M_xx = f->one_pass ? f->gbuf + ((size_t)kv * c.L_src + sl) * N * N : G.M_xx + (size_t)j * N * N;
                v.M_xy = G.M_xy + (size_t)j * N * G.q;
                views.push_back(v);
                out.push_back(f->r2 + (((size_t)kv * c.L_src + sl) * c.L_tgt + f->t0) * H);
            }
        std::vector<const kvmap_gram_state*> st;
        for (const auto& v : views) st.push_back(&v);
        FIT_TRY(kvmap_ridge_r2_batch(f->ctx, st.data(), (int)st.size(), c.lambda, c.head_dim, out.data(), s));
        if (f->pass == f->sel_passes - 1) {
            double* scores = c.scores ? c.scores : f->own_scores;
            FIT_HIP(launch_fit_select(f->r2, c.L_src, c.L_tgt, H, c.k, scores, c.layer_sel, s));
            FIT_HIP(hipMemcpyAsync(f->sel.data(), c.layer_sel, f->sel.size() * sizeof(int32_t),
                                   hipMemcpyDeviceToHost, s));
            FIT_HIP(hipStreamSynchronize(s));
            if (f->one_pass) FIT_TRY(solve_maps_from_full(f, s));
            free_stage(f);
        }
        return KVMAP_OK;
    }
    const size_t es = esize(c.out_dtype);
    std::vector<const kvmap_gram_state*> st;
    std::vector<void*> Ws, bs;
    for (int t = f->t0; t < f->t1; ++t)
        for (int kv = 0; kv < 2; ++kv) {
            st.push_back(&f->states[2 * (t - f->t0) + kv]);
            Ws.push_back((char*)(kv ? c.W_v : c.W_k) + (size_t)t * f->N * f->F * es);
            bs.push_back((char*)(kv ? c.b_v : c.b_k) + (size_t)t * f->N * es);
        }
    FIT_TRY(kvmap_ridge_solve_device_batch(f->ctx, st.data(), (int)st.size(), c.lambda, Ws.data(), bs.data(),
                                           c.out_dtype, s));
    if (f->pass == f->sel_passes + f->map_passes - 1) free_stage(f);
    return KVMAP_OK;
}

void destroy(kvmap_fit* f) {
    if (!f) return;
    FitDevice g(f->device);
    (void)hipDeviceSynchronize();
    free_stage(f);
    (void)hipFree(f->r2);
    (void)hipFree(f->own_scores);
    (void)hipFree(f->xrows);
    (void)hipFree(f->yrows);
    for (int kv = 0; kv < 2; ++kv) {
        (void)hipFree(f->accx[kv]);
        (void)hipFree(f->accy[kv]);
    }
    (void)hipFree(f->gbuf);
    delete f;
}

}  // namespace

extern "C" int kvmap_fit_create(kvmap_ctx* ctx, const kvmap_fit_config* cfg, kvmap_fit** out) {
    if (!out) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: out is NULL");
    *out = nullptr;
    if (!ctx || !cfg) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: ctx or cfg is NULL");
    const kvmap_fit_config& c = *cfg;
    if (c.head_dim != 64 && c.head_dim != 128)
        return report(KVMAP_ERR_UNSUPPORTED, "kvmap_fit_create: head_dim %d (64 or 128 supported)", (int)c.head_dim);
    if (c.L_src < 1 || c.L_src > kMaxFitSrcLayers || c.L_tgt < 1 || c.H_kv < 1 || c.k < 1 || c.k > c.L_src)
        return report(KVMAP_ERR_SHAPE, "kvmap_fit_create: L_src=%d (1..%d), L_tgt=%d, H_kv=%d, k=%d out of range",
                      (int)c.L_src, kMaxFitSrcLayers, (int)c.L_tgt, (int)c.H_kv, (int)c.k);
    const int64_t N = (int64_t)c.H_kv * c.head_dim, F = N * c.k;
    if (F > kMaxGramWidth || c.k > kMaxRowLayers)
        return report(KVMAP_ERR_SHAPE, "kvmap_fit_create: k*H*d = %lld exceeds %d (or k > %d)", (long long)F,
                      kMaxGramWidth, kMaxRowLayers);
    for (int32_t dt : {c.dtype, c.out_dtype})
        if (dt != KVMAP_DTYPE_BF16 && dt != KVMAP_DTYPE_F32)
            return report(KVMAP_ERR_UNSUPPORTED, "kvmap_fit_create: dtype %d unknown", (int)dt);
    for (int side = 0; side < 2; ++side) {
        const double theta = side ? c.theta_tgt : c.theta_src;
        const double* f = side ? c.inv_freq_tgt : c.inv_freq_src;
        if (f) {
            for (int i = 0; i < c.head_dim / 2; ++i)
                if (!(f[i] >= 0.0) || !std::isfinite(f[i]))
                    return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: inv_freq[%d] must be finite and >= 0", i);
        } else if (!(theta > 0.0) || !std::isfinite(theta)) {
            return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: RoPE bases must be finite and > 0");
        }
    }
    if (!(c.lambda >= 0.0) || !std::isfinite(c.lambda))
        return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: lambda must be finite and >= 0");
    const int max_sel_block = (int)std::min<int64_t>(kMaxRowLayers, kMaxGramWidth / N);
    if (c.select_block < 0 || c.select_block > max_sel_block || c.map_block < 0)
        return report(KVMAP_ERR_SHAPE, "kvmap_fit_create: select_block %d (0..%d), map_block %d", (int)c.select_block,
                      max_sel_block, (int)c.map_block);
    if (!c.layer_sel || !c.W_k || !c.b_k || !c.W_v || !c.b_v)
        return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: NULL output");
    if (((uintptr_t)c.layer_sel | (uintptr_t)c.W_k | (uintptr_t)c.b_k | (uintptr_t)c.W_v | (uintptr_t)c.b_v) & 3)
        return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: outputs must be 4-byte aligned");
    if (((uintptr_t)c.scores) & 7)
        return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_create: scores must be 8-byte aligned");
    const int dev = context_device(ctx);
    FitDevice g(dev);
    kvmap_fit* f = new kvmap_fit;
    f->ctx = ctx;
    f->cfg = c;
    f->device = dev;
    f->N = (int)N;
    f->F = (int)F;
    f->sel.assign((size_t)c.L_tgt * c.k, 0);
    if (c.inv_freq_src) f->freq_src.assign(c.inv_freq_src, c.inv_freq_src + c.head_dim / 2);
    if (c.inv_freq_tgt) f->freq_tgt.assign(c.inv_freq_tgt, c.inv_freq_tgt + c.head_dim / 2);
    f->cfg.inv_freq_src = nullptr;  // the copies above are used from here on
    f->cfg.inv_freq_tgt = nullptr;
    f->sel_block = c.select_block ? c.select_block : std::min<int>(c.L_tgt, max_sel_block);
    f->map_block = c.map_block ? std::min<int>(c.map_block, c.L_tgt) : c.L_tgt;
    f->sel_passes = c.given_sel ? 0 : (c.L_tgt + f->sel_block - 1) / f->sel_block;
    f->map_passes = (c.L_tgt + f->map_block - 1) / f->map_block;
    f->group = (int)std::min<int64_t>(std::min<int64_t>(c.L_src, kMaxGramWidth / N), kMaxRowLayers);
    f->groups = (c.L_src + f->group - 1) / f->group;
    // one pass: one source group, one target block, and the choice not forced off
    f->one_pass = !c.given_sel && f->groups == 1 && f->sel_passes == 1 && !c.two_pass;
    if (f->one_pass) f->map_passes = 0;
    int st = KVMAP_OK;
    if (c.given_sel) {
        hipError_t e = hipMemcpy(f->sel.data(), c.layer_sel, f->sel.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
        if (e != hipSuccess) st = report(KVMAP_ERR_DEVICE, "kvmap_fit_create: reading layer_sel: %s", hipGetErrorString(e));
        for (int t = 0; t < c.L_tgt && st == KVMAP_OK; ++t) {
            std::vector<char> seen(c.L_src, 0);
            for (int j = 0; j < c.k && st == KVMAP_OK; ++j) {
                const int v = f->sel[(size_t)t * c.k + j];
                if (v < 0 || v >= c.L_src || seen[v])
                    st = report(KVMAP_ERR_SHAPE, "kvmap_fit_create: layer_sel[%d][%d] = %d out of range or repeated", t,
                                j, v);
                else
                    seen[v] = 1;
            }
        }
    } else {
        hipError_t e = hipMalloc((void**)&f->r2, (size_t)2 * c.L_src * c.L_tgt * c.H_kv * sizeof(double));
        if (e == hipSuccess && !c.scores) e = hipMalloc((void**)&f->own_scores, (size_t)c.L_tgt * c.L_src * sizeof(double));
        if (e != hipSuccess)
            st = report(e == hipErrorOutOfMemory ? KVMAP_ERR_OUT_OF_MEMORY : KVMAP_ERR_DEVICE,
                        "kvmap_fit_create: %s", hipGetErrorString(e));
    }
    if (st != KVMAP_OK) {
        destroy(f);
        return st;
    }
    *out = f;
    return report(KVMAP_OK, "%s", "");
}

extern "C" int kvmap_fit_next_pass(kvmap_fit* f, kvmap_fit_pass* info, void* stream) {
    if (!f || !info) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_next_pass: NULL argument");
    FitDevice g(f->device);
    hipStream_t s = (hipStream_t)stream;
    const int passes = f->sel_passes + f->map_passes;
    if (f->pass >= passes) {
        *info = kvmap_fit_pass{0, 0, 0, passes, passes};
        return report(KVMAP_OK, "%s", "");
    }
    if (f->pass >= 0) FIT_TRY(close_pass(f, s));
    ++f->pass;
    if (f->pass >= passes) {
        f->stage = 0;
        *info = kvmap_fit_pass{0, 0, 0, passes, passes};
        return report(KVMAP_OK, "%s", "");
    }
    FIT_TRY(open_pass(f, s));
    *info = kvmap_fit_pass{f->stage, f->t0, f->t1, f->pass, passes};
    return report(KVMAP_OK, "%s", "");
}

extern "C" int kvmap_fit_add(kvmap_fit* f, const void* src_k, const void* src_v, const void* tgt_k,
                             const void* tgt_v, int64_t T, int64_t pos0, void* stream) {
    if (!f) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_add: fit is NULL");
    if (f->stage == 0) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_add: no pass is open");
    if (!src_k || !src_v || !tgt_k || !tgt_v) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_add: NULL cache");
    if (T < 1 || T > (int64_t(1) << 31)) return report(KVMAP_ERR_SHAPE, "kvmap_fit_add: T=%lld out of range", (long long)T);
    if (pos0 < 0) return report(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_fit_add: pos0 < 0");
    const kvmap_fit_config& c = f->cfg;
    FitDevice g(f->device);
    hipStream_t s = (hipStream_t)stream;
    const size_t es = esize(c.dtype);
    const int d = c.head_dim, H = c.H_kv;
    const kvmap_rope rs{c.theta_src, pos0, KVMAP_ROPE_HALF_SPLIT, f->freq_src.empty() ? nullptr : f->freq_src.data()};
    const kvmap_rope rt{c.theta_tgt, pos0, KVMAP_ROPE_HALF_SPLIT, f->freq_tgt.empty() ? nullptr : f->freq_tgt.data()};
    const void* src[2] = {src_k, src_v};
    const void* tgt[2] = {tgt_k, tgt_v};
    if (f->stage == 1 && f->groups == 1 && T <= kAccRows) {
        // gather this sequence's rows behind the ones already accumulated; merge when full
        const int nb = f->t1 - f->t0;
        const size_t xrow = (size_t)f->group * f->N * es, yrow = (size_t)nb * f->N * es;
        if (f->accx_cap < (size_t)kAccRows * xrow || f->accy_cap < (size_t)kAccRows * yrow) {
            FIT_TRY(flush_rows(f, s));
            FIT_HIP(hipStreamSynchronize(s));
            size_t cx = 0, cy = 0;
            for (int kv = 0; kv < 2; ++kv) {
                cx = f->accx_cap;
                cy = f->accy_cap;
                FIT_TRY(ensure_rows(&f->accx[kv], &cx, (size_t)kAccRows * xrow, s));
                FIT_TRY(ensure_rows(&f->accy[kv], &cy, (size_t)kAccRows * yrow, s));
            }
            f->accx_cap = cx;
            f->accy_cap = cy;
        }
        if (f->n_acc + T > kAccRows) FIT_TRY(flush_rows(f, s));
        std::vector<int32_t> block(nb), layers(c.L_src);
        for (int j = 0; j < nb; ++j) block[j] = f->t0 + j;
        for (int j = 0; j < c.L_src; ++j) layers[j] = j;
        for (int kv = 0; kv < 2; ++kv) {
            FIT_TRY(kvmap_cache_rows(f->ctx, tgt[kv], c.L_tgt, H, T, d, c.dtype, block.data(), nb, kv ? nullptr : &rt,
                                     (char*)f->accy[kv] + (size_t)f->n_acc * yrow, s));
            FIT_TRY(kvmap_cache_rows(f->ctx, src[kv], c.L_src, H, T, d, c.dtype, layers.data(), c.L_src,
                                     kv ? nullptr : &rs, (char*)f->accx[kv] + (size_t)f->n_acc * xrow, s));
        }
        f->n_acc += T;
    } else if (f->stage == 1) {
        const int nb = f->t1 - f->t0;
        FIT_TRY(ensure_rows(&f->xrows, &f->xcap, (size_t)T * f->group * f->N * es, s));
        FIT_TRY(ensure_rows(&f->yrows, &f->ycap, (size_t)T * nb * f->N * es, s));
        std::vector<int32_t> block(nb);
        for (int j = 0; j < nb; ++j) block[j] = f->t0 + j;
        for (int kv = 0; kv < 2; ++kv) {
            FIT_TRY(kvmap_cache_rows(f->ctx, tgt[kv], c.L_tgt, H, T, d, c.dtype, block.data(), nb, kv ? nullptr : &rt,
                                     f->yrows, s));
            for (int g = 0; g < f->groups; ++g) {
                const int gl = group_layers(f, g);
                std::vector<int32_t> layers(gl);
                for (int j = 0; j < gl; ++j) layers[j] = g * f->group + j;
                FIT_TRY(kvmap_cache_rows(f->ctx, src[kv], c.L_src, H, T, d, c.dtype, layers.data(), gl,
                                         kv ? nullptr : &rs, f->xrows, s));
                FIT_TRY(kvmap_gram(f->ctx, f->xrows, f->yrows, T, c.dtype, &f->states[kv * f->groups + g], s));
            }
        }
    } else {
        FIT_TRY(ensure_rows(&f->xrows, &f->xcap, (size_t)T * f->F * es, s));
        FIT_TRY(ensure_rows(&f->yrows, &f->ycap, (size_t)T * f->N * es, s));
        for (int32_t t = f->t0; t < f->t1; ++t)
            for (int kv = 0; kv < 2; ++kv) {
                FIT_TRY(kvmap_cache_rows(f->ctx, src[kv], c.L_src, H, T, d, c.dtype, &f->sel[(size_t)t * c.k], c.k,
                                         kv ? nullptr : &rs, f->xrows, s));
                FIT_TRY(kvmap_cache_rows(f->ctx, tgt[kv], c.L_tgt, H, T, d, c.dtype, &t, 1, kv ? nullptr : &rt,
                                         f->yrows, s));
                FIT_TRY(kvmap_gram(f->ctx, f->xrows, f->yrows, T, c.dtype, &f->states[2 * (t - f->t0) + kv], s));
            }
    }
    f->n_pass += T;
    return report(KVMAP_OK, "%s", "");
}

extern "C" int kvmap_fit_destroy(kvmap_fit* f) {
    destroy(f);
    return report(KVMAP_OK, "%s", "");
}
