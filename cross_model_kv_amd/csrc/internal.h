// Internal launch interface shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct kvmap_ctx;

namespace kvmap {

// Element storage types.
enum class Elem : int { BF16 = 0, F32 = 1 };

// Geometry of one apply call, in the notation of include/kvmap.h.
struct ApplyGeom {
    int L_src, L_tgt, H, d, k;
    int64_t T;
    int F() const { return k * H * d; }
    int N() const { return H * d; }
};

// ---- RoPE tables / key de-rotation (rope.hip) -------------------------------------
// Rotary frequencies of one model: f_i = theta^(-2i/d) (formed on the device), or the given
// list (the model's own factors); passed by value.
struct RopeFreqs {
    double theta;
    int given;       // nonzero: f[0 .. d/2) are the frequencies
    double f[64];
};

// tab[t][i] = (cos a, sin a), a = (pos0 + t) * f_i, formed in float64.
hipError_t launch_rope_table(float2* tab, int64_t T, int d, const RopeFreqs& fr, int64_t pos0, hipStream_t s);

// tab[t][i] = (cos A, sin A), A = (pos0_s + t) f_s,i - (pos0_t + t) f_t,i, formed in float64:
// rotating by -A re-encodes a source-roped key to the target RoPE.
hipError_t launch_rope_diff_table(float2* tab, int64_t T, int d, const RopeFreqs& fs, int64_t pos0_s,
                                  const RopeFreqs& ft, int64_t pos0_t, hipStream_t s);
// ws[l][h][t][:] = every pair of src[l][h][t][:] rotated by -a (a from tab), for every l in
// layers[0..n_layers).
hipError_t launch_derope(Elem e, const void* src, void* ws, const int32_t* layers, int n_layers,
                         const ApplyGeom& g, const float2* tab, hipStream_t s);

// rows[t][(j*H + h)*d + e] = src[layers[j]][h][t][e], stripped with tab when tab != NULL.
constexpr int kMaxRowLayers = 128;
struct RowLayers {
    int32_t l[kMaxRowLayers];
};
hipError_t launch_rows(Elem e, const void* src, void* out, const RowLayers& layers, int n_layers, int H,
                       int64_t T, int d, const float2* tab, hipStream_t s);

// ---- map GEMMs (gemm_bf16.hip, gemm_f32.hip) ----------------------------------------
struct MapArgs {
    const void* xk;     // de-rotated source keys [L_src][H][T][d]
    const void* xv;     // source values          [L_src][H][T][d]
    const int32_t* sel; // device [L_tgt][k]
    const void* Wk; const void* bk;
    const void* Wv; const void* bv;
    const float2* tab_tgt;  // [T][d/2]
    void* outk; void* outv;
};
hipError_t launch_map_bf16(const MapArgs& a, const ApplyGeom& g, int cus, hipStream_t s);
hipError_t launch_map_f32(const MapArgs& a, const ApplyGeom& g, hipStream_t s);

// Short caches (gemm_bf16_small.hip): bf16 applies with T <= kSmallT tokens take the persistent
// short-cache kernel (fp32 partial sums in `part`, then a deterministic reduce with bias and
// target RoPE; with an unsplit K reduction at 33 to 128 tokens the kernel finishes the rows
// itself); measured faster than the long-cache kernel up to 128 tokens.
#ifndef KVMAP_SMALL_T
#define KVMAP_SMALL_T 128
#endif
constexpr int64_t kSmallT = KVMAP_SMALL_T;
struct SmallPlan {
    int nN, nP, KS, kps;  // feature tiles, token tiles, K splits, K-steps per split
    int n_items, grid;    // work items (tiles x splits), persistent workgroups
    bool fused;           // items finish in the kernel (no partial sums, no reduce kernel)
    size_t part_bytes;    // fp32 partial sums [KS][L_tgt][2][T][N]; 0 when fused
};
SmallPlan map_bf16_small_plan(const ApplyGeom& g, int cus);
hipError_t launch_map_bf16_small(const MapArgs& a, const ApplyGeom& g, const SmallPlan& pl, float* part,
                                 hipStream_t s);

// Count of non-finite elements (bf16 or f32) added atomically into *count.
hipError_t launch_count_nonfinite(Elem e, const void* p, int64_t n, unsigned int* count,
                                  hipStream_t s);

// ---- fit-side statistics (gram.hip) ------------------------------------------------
struct GramScratch {
    float* part;   // [splits][p + q] partial column sums
    float* part2;  // [splits][p + q] partial column sums of squares (y of a state with ss_y)
    float* cx;     // [p]  batch shift (fp32 column mean of x)
    float* cy;     // [q]
    float* mx;     // [p]  mean of (x - cx) over the batch (tiny correction)
    float* my;     // [q]
    float* dx;     // [p]  delta = batch mean - running mean
    float* dy;     // [q]
    uint16_t* split;  // bf16 path: [p + q][ceil(n_b / 32)][64] shifted, split, transposed batch
    int splits;       // row splits of the column sums
    int max_splits;   // rows of `part`
};
// Sizes (floats) of the scratch for p, q.
size_t gram_scratch_floats(int p, int q, int splits);
// bd > 0: M_xx is kept only on its p / bd diagonal blocks of bd x bd, stored compactly
// ([p / bd][bd][bd]); 0: the whole p x p matrix.
hipError_t launch_gram_batch(Elem e, const void* X, const void* Y, int64_t n_b, int p, int q,
                             int64_t n_old, float* mean_x, float* mean_y, float* M_xx,
                             float* M_xy, float* ss_y, int bd, const GramScratch& sc, hipStream_t s);
// Rows per kvmap_gram sub-batch: larger batches are merged in pieces of at most this many
// rows (the split operands' scratch and 32-bit tile offsets are sized for it).
constexpr int64_t kGramSubBatch = 16384;
// Bytes of the static device scratch of kvmap_gram_noalloc (one array per GPU).
#define KVMAP_STATIC_SCRATCH_BYTES (size_t(64) << 20)
size_t gram_split_elems(int p, int q, int64_t n_b);  // uint16 elements of `split` for n_b rows
int gram_split_blocks(int64_t n_b, int max_splits);
// c: the shift per column (bf16 values), or with round_c any fp32 values rounded to bf16 here.
hipError_t launch_gram_split(const void* A, int64_t n_b, int cols, const float* c, int round_c, uint16_t* S,
                             float* part, int part_stride, int col_off, float* part2, int splits, hipStream_t s);
hipError_t launch_gram_x3(const uint16_t* Sx, const uint16_t* Sy, int64_t n_b, int p, int q, const float* mx,
                          const float* my, const float* dx, const float* dy, float coef, int fresh,
                          float* M_xx, float* M_xy, int bd, hipStream_t s);
hipError_t launch_gram_merge(int p, int q, int64_t n_dst, int64_t n_src, float* mean_x,
                             float* mean_y, float* M_xx, float* M_xy, float* ss_y, const float* s_mean_x,
                             const float* s_mean_y, const float* s_M_xx, const float* s_M_xy, const float* s_ss_y,
                             int bd, const GramScratch& sc, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

// ---- ridge solve on the device (ridge_dev.hip), float64 --------------------------------
// Up to kRidgeMaxBatch independent systems of one (p, q) are solved together: every kernel of
// the factorisation and the substitutions covers all of them (grid y = system), so the serial
// chain of 64-wide block steps is paid once per batch.
constexpr int kRidgeMaxBatch = 16;
struct RidgeSys {
    const float* M_xx;
    const float* M_xy;
    const float* mean_x;  // solve: b = mean_y - mean_x W
    const float* mean_y;
    const float* ss_y;    // R^2: total sums of squares
    void* W_out;          // solve: [q][p] output-major, bf16 or fp32
    void* b_out;          // solve: [q]
    double* r2_out;       // R^2: [q / group]
};
// Scratch for n systems (fp64 factor, right-hand sides, residual sums; pivot flags at the end).
size_t ridge_dev_scratch_bytes(int p, int q, int n);
// Pivot flags of the n systems (nonzero: not positive definite) inside that scratch.
int* ridge_dev_flags(void* scratch, int p, int q, int n);
// A side stream (default priority) and events for the lookaheads: the bulk of each panel's
// trailing update (and, in the back substitution, of its update of the rows above) runs there,
// overlapping the next panel's chain on the caller's stream.  side NULL: everything on the
// caller's stream.
// A second one takes each factored panel's forward substitution.
struct RidgeOverlap {
    hipStream_t side;
    hipEvent_t main_ready;  // recorded on the caller's stream, waited on by the side stream
    hipEvent_t side_done;   // recorded on the side stream, waited on by the caller's stream
    hipEvent_t side_done2;  // a second one: the back substitution alternates between the two
    hipStream_t fwd;        // NULL: the forward substitution runs after the factorisation
    hipEvent_t fwd_ready;   // recorded on the caller's stream after each panel, waited on by fwd
    hipEvent_t fwd_done;    // recorded on fwd after the last panel, waited on by the caller's stream
};
hipError_t launch_ridge_dev(int n, int p, int q, const RidgeSys* sys, double lambda, bool bf16, void* scratch,
                            hipStream_t s, const RidgeOverlap& ov);
// r2_out[g] = in-sample R^2 of the ridge fit pooled over y columns g*group .. +group-1
hipError_t launch_ridge_r2(int n, int p, int q, const RidgeSys* sys, double lambda, int group, void* scratch,
                           hipStream_t s, const RidgeOverlap& ov);

// ---- fit driver's scoring kernel (fit.hip) ----------------------------------------------
// scores[t][s] = mean over {K, V} and heads of r2[kv][s][t][h]; sel[t] = the k best s, ties to
// the lower index, ascending.
hipError_t launch_fit_select(const double* r2, int L_src, int L_tgt, int H, int k, double* scores,
                             int32_t* sel, hipStream_t s);

// Error reporting shared by the C-ABI files: sets the calling thread's last-error string.
int report(int status, const char* fmt, ...);
// HIP device a context is bound to (-1 for NULL).
int context_device(const struct ::kvmap_ctx* c);

}  // namespace kvmap

#include "ridge.h"
