// Internal declarations of libigconv: error reporting and the kernel
// launchers the C entry points and decoder_forward share. Launchers assume
// their arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ig_conv.h"

namespace ig {

// Record the reason for a failure on this thread and return `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread's last error.
void clear_error();
// IG_EHIP with the HIP error's text when the last launch failed, else IG_OK.
int check_launch(const char *what);

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------
// implicit GEMM (MFMA f16 -> f32)
// ---------------------------------------------------------------------
enum GemmMode { kGemm = 0, kConv3x3 = 1, kConv3x3Up2 = 2 };
// The 3x3 conv kernels address their f16 input with 32-bit byte offsets
// and mark out-of-image patch pixels with an offset past every input: the
// input must stay below this many bytes.
constexpr int64_t kConvInMaxBytes = 0x7fff0000;
// widest padded channel count a conv takes (its weight plane stays below
// 2 GB and a stage's channel offset below 64 KB)
constexpr int kConvMaxChannels = 8192;

struct IgemmArgs {
    const _Float16 *a;  // kGemm: A [M][lda]; convs: NHWC image [H*W][cin_p]
    const _Float16 *b;  // B [N][ldb] (conv plane: ldb = taps * cin_p)
    const float *bias;  // [N] or null
    void *c;            // [M][ldc], f32 or f16
    int M, N, K;
    int lda, ldb, ldc;
    int H, W;           // input image (convs); the up2 output is 2H x 2W
    int cin_p;
    float oscale;
    int accumulate;     // f32 output only: c += result
    int out_f16;
    // 3x3 convs whose tile spans all N channels: the epilogue can also
    // emit the per-pixel RMS_norm of the result (pages' RMSN_SRC) as f16
    // into ny [M][N]: v * sqrt(norm_c) / max(|v|, norm_eps) * gamma, then
    // SiLU if norm_silu; with write_out = 0 the f32 result is not stored
    const float *ngamma;  // [N], or null for no norm
    _Float16 *ny;
    int norm_c, norm_silu;
    float norm_eps;
    int write_out = 1;
    // 3x3 convs without the norm: the epilogue can also emit the guarded
    // f16 copy f16(v * gscale) of the (accumulated) f32 result v into
    // yg [M][ldc] -- the cast of the stream before an up conv
    _Float16 *yg = nullptr;
    float gscale = 1.f;
    // 3x3 convs without the norm: with gn_part set, the epilogue also
    // writes GroupNorm statistics of the (accumulated) f32 result v: for
    // every pixel tile pt (16 x 32 output pixels, row-major over the frame)
    // and group g of gn_cpg consecutive real channels (< gn_creal), the
    // tile's (count, mean, M2) at gn_part[(g * gn_nchunk + pt) * 3]; gn_cpg
    // divides 64 and is a multiple of 4 (conv_gn_stats_supported)
    float *gn_part = nullptr;
    int gn_cpg = 0, gn_creal = 0, gn_nchunk = 0;
    // measurement: when set, the weight-stationary conv's first wave
    // writes the shader-clock and real-time counters at its start and end
    // (clk[0], clk[1], clk[2], clk[3])
    unsigned long long *clk = nullptr;
};

// Launch the MFMA implicit GEMM for `mode`; picks the tile shape. The 3x3
// modes go to the patch-reusing convolution kernel.
void launch_igemm(int mode, const IgemmArgs &a, hipStream_t s);
// The 3x3 convolutions (kConv3x3, kConv3x3Up2) with per-tile input patches.
// With a.ngamma set, N must be 64 or 128 and accumulate 0. Shapes that
// conv_ws_supported accepts go to launch_conv_ws.
void launch_conv_halo(int mode, const IgemmArgs &a, hipStream_t s);
// The 3x3 convolutions at cin_p = N = ldc = 128 with the weights held in
// registers; true when the shape fits (it depends on the channels and the
// output width, not the height, so bands and whole frames agree).
bool conv_ws_supported(int mode, const IgemmArgs &a);
// GroupNorm statistics from the conv's epilogue: the pixel tiles of a 3x3
// conv's output (the partials' chunk count), and whether groups of cpg
// channels out of c_real, padded to cout_p, can be gathered there
int conv_gn_chunks(int mode, int H, int W);
bool conv_gn_stats_supported(int cout_p, int c_real, int groups);
void launch_conv_ws(int mode, const IgemmArgs &a, hipStream_t s);
// The buffer later launches of the weight-stationary conv record their
// clock counters in (null: none).
void set_clock_probe(void *buf);

// ---------------------------------------------------------------------
// plain NT GEMM C = oscale * A.B^T with the attention's softmax epilogues
// ---------------------------------------------------------------------
enum GemmEpi { kEpiF32 = 0, kEpiF16 = 1, kEpiStats = 2, kEpiProb = 3 };

struct Gemm2Args {
    const _Float16 *a;     // A [M][lda]
    const _Float16 *b;     // B [N][ldb]
    void *c;               // C [M][ldc]: f32 (kEpiF32), f16 (kEpiF16, kEpiProb)
    const float *bias;     // [N] or null (kEpiF32, kEpiF16)
    float *stats;          // kEpiStats: [M][gemm2_stat_parts(N)] (max, sum) pairs
    const float *rowstat;  // kEpiProb: [M] (max, 1 / sum) pairs
    int M, N, K;
    int lda, ldb, ldc;
    int valid;             // kEpiStats, kEpiProb: columns >= valid are masked
    int accumulate;        // kEpiF32: C += result
    float oscale;
    // a pair of products sharing A in one launch (kEpiF32, kEpiF16): with
    // nsplit > 0, columns [nsplit, N) use b2 [N - nsplit][ldb], c2 and bias2
    // (column n - nsplit); nsplit must be a multiple of 256
    const _Float16 *b2 = nullptr;
    void *c2 = nullptr;
    const float *bias2 = nullptr;
    int nsplit = 0;
};

// true when the shapes, strides and alignment fit k_gemm2 (K % 64 == 0,
// N % 64 == 0, 16-byte rows and pointers, operands below 3.75 GiB)
bool gemm2_supported(const Gemm2Args &a);
void launch_gemm2(int epi, const Gemm2Args &a, hipStream_t s);
// partial statistics per row that kEpiStats writes for N columns
int gemm2_stat_parts(int N);
// rowstat[r] = (max, 1 / sum) from the partial statistics of row r
void launch_rowstat(const float *stats, int nparts, int rows, float *rowstat, hipStream_t s);

// single-pass attention core (C = 128, 256, 384 or 512):
// out = f16(softmax(q k^T / sqrt(C)) v + bv)
struct FlashArgs {
    const _Float16 *q, *k;  // [ld][C] rows (rows >= m are read, never used)
    const _Float16 *vt;     // V^T [C][ld]
    int ld;                 // rows of q and k; row stride of V^T
    int m;                  // queries = keys
    int c;                  // head width
    float scale_log2;       // log2(e) / sqrt(C)
    const float *bv;        // [C] or null
    _Float16 *out;          // [m][C]
    int nsplit, bps;        // key ranges and 32-key blocks per range (set by the launcher)
    float *opart, *ml;      // per range: partial O [m][C] and (max, sum) [m] (workspace)
};
bool flash_supported(int m, int ld, int c);
size_t flash_workspace_bytes(int m, int c);
void launch_flash(FlashArgs a, void *ws, hipStream_t s);

// ---------------------------------------------------------------------
// memory-bound kernels
// ---------------------------------------------------------------------
// RMS_norm (+ bias on read, + SiLU) -> f16 y; with yg, also the guarded
// cast f16((x + bias) * 2^-guard_log2) of the same rows -> yg
void launch_rmsnorm(const float *x, int M, int cp, int c_real, const float *bias,
                    const float *gamma, int silu, float eps, _Float16 *y, hipStream_t s,
                    _Float16 *yg = nullptr, int guard_log2 = 0);
// GroupNorm: workspace for the per-chunk statistics, support check, launch
size_t gn_workspace_bytes(int M, int cp, int groups);
bool gn_supported(int cp, int c_real, int groups);
// The device address of the GroupNorm scratch array on the current device
// (looked up once per device; null on failure) and its size in bytes.
void *gn_scratch_ptr();
size_t gn_scratch_bytes();
void launch_groupnorm(const float *x, int M, int cp, int c_real, int groups, const float *bias,
                      const float *gamma, const float *beta, int silu, float eps, void *ws, _Float16 *y,
                      hipStream_t s);
// GroupNorm of x whose group statistics came as nchunk partial (count,
// mean, M2) per group in part [groups][nchunk][3] (a conv epilogue's): the
// final merge and the apply pass only (x is read once). tab: 3 cp floats,
// 16-byte aligned, for the per-channel offset, scale and shift.
void launch_groupnorm_partials(const float *x, int M, int cp, int c_real, int groups, const float *gamma,
                               const float *beta, int silu, float eps, const float *part, int nchunk, float *tab,
                               _Float16 *y, hipStream_t s);
void launch_guard_cast(const float *x, int M, int C, const float *bias, int guard_log2,
                       _Float16 *y, hipStream_t s);
void launch_combine(float *x, const float *h, const float *hb, const float *sv, const float *sb,
                    int M, int C, int mode, hipStream_t s);
void launch_softmax(const float *S, int rows, int lds, int valid, int ncols, _Float16 *P, int ldp,
                    hipStream_t s);
void launch_latent_ingest(const float *z, int zc, int M, int cp, _Float16 *y, hipStream_t s);
// out[ch][p] = y[p][ch] (+ bias[ch]) for p < M, output planes HWo apart
// (HWo <= 0: M)
void launch_nhwc_to_nchw(const float *y, int M, int ld, int nch, const float *bias, float *out,
                         hipStream_t s, int64_t HWo = 0);
void launch_pack_weights(const _Float16 *w, int cout, int cin, int k, int cout_p, int cin_p,
                         _Float16 *plane, hipStream_t s);
// the decoder's output conv into the NCHW frame; by default the whole
// image, else rows r0 .. r1 - 1 of it with output planes HWo apart (out
// points at the frame pixel of image row 0)
void launch_conv_out(const _Float16 *x, int H, int W, int cin_p, const _Float16 *plane, int cout, int cout_p,
                     const float *bias, float *out, hipStream_t s, int r0 = 0, int r1 = -1, int64_t HWo = 0);
void launch_zero_rows_f16(_Float16 *y, int r0, int r1, int ld, hipStream_t s);
void launch_dupup(const float *src, int H, int W, int cin_p, float *x, int cout, int cout_p,
                  int factor, int repeats, int ft, hipStream_t s);

}  // namespace ig
