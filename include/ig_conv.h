/*
 * ig_conv.h -- C ABI of libigconv, the MI355X (gfx950) implementation of
 * the resident image-VAE decoder's NHWC implicit-GEMM convolution path.
 *
 * Source pages (cited by title and item):
 *   [QI]  "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs" -- the resident
 *         decoder: module doc, RMSN_SRC, CAST_SRC, OUT_SRC, `guard`,
 *         `cpad`, `qconv`, `Rec::conv`/`conv_s`/`rmsn`/`combine`/`cast`/
 *         `resnet`, `attention`, `run_blocks`, `output_rows`, `decode`.
 *   [VAE] "cortiq-engine 0.7.6, src/vae.rs" -- the CPU NCHW decoder:
 *         `Conv2d::apply`, `upsample2x`, `AttnBlock::apply`,
 *         `VaeDecoder::decode`.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer the caller allocated and
 *     owns; the library keeps none of them after the call returns.
 *     f16 data is IEEE binary16, passed as uint16_t bit patterns.
 *     Every f16/f32 buffer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls are
 *     asynchronous on it; results are ready when the stream is.
 *   - Activations are NHWC: pixel-major rows, channels contiguous,
 *     rows [M][cp] with cp the padded channel count. Padded channels hold
 *     zeros; weights and norm scales are zero there, so outputs in the pad
 *     stay zero ([QI] module doc and `cpad`: channels padded to multiples
 *     of 64).
 *   - Return value: IG_OK (0) or a negative status. Shapes and pointers are
 *     checked BEFORE anything is enqueued: on IG_EINVAL / IG_EUNSUPPORTED /
 *     IG_EWORKSPACE nothing was enqueued and no output was touched (the
 *     pages' "declined, output untouched" contract of [QI] `decode` and
 *     `decline`). IG_EHIP means a launch failed after validation.
 *     ig_last_error() returns the reason as text (per thread).
 *   - M = 0 (no pixels / rows) is valid and enqueues nothing.
 */
#ifndef IG_CONV_H
#define IG_CONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IG_OK 0
#define IG_EINVAL (-1)       /* bad argument: null or misaligned pointer, bad size */
#define IG_EUNSUPPORTED (-2) /* a shape outside the kernels' contract */
#define IG_EWORKSPACE (-3)   /* workspace missing or too small */
#define IG_EHIP (-4)         /* a HIP launch or runtime call failed */

#define IG_MAX_RES 4 /* resnet units per up stage */
#define IG_MAX_UP 8  /* up stages */
/* the decoder's norm (ig_decoder.norm_kind): */
#define IG_NORM_RMS 0   /* RMS_norm, x / max(|x|, 1e-12) sqrt(C) gamma ([QI] RMSN_SRC) */
#define IG_NORM_GROUP 1 /* GroupNorm(norm_groups, norm_eps) with gamma and beta ([VAE] GroupNorm) */

/* Text of the last error on the calling thread ("" if none). */
const char *ig_last_error(void);

/* Library version, (major << 16) | minor. */
int ig_version(void);

/* ---------------------------------------------------------------------
 * Weight packing ([QI] `qconv`: the f16 "plane" of a conv, zero padded,
 * K ordered (tap, channel) with tap = ky*3 + kx). From an OIHW f16 weight
 * w[cout][cin][k][k]:
 *   k = 1: plane[o][ci] = w[o][ci][0][0]                 -- [cout_p][cin_p]
 *   k = 3: plane[c][tap][o][e] = w[o][16c + e][ky][kx]    -- [cin_p/16][9][cout_p][16]
 * zero for o >= cout or channel >= cin. The 3x3 layout keeps, for each
 * 16-channel slice and tap, the 16 weights of every output channel
 * together, so a convolution stage reads its weights as one contiguous
 * block; the plane holds the same numbers as the pages' [cout_p][9][cin_p].
 * cout_p >= cout, cin_p >= cin, both multiples of 64.
 * --------------------------------------------------------------------- */
int ig_pack_conv_weights(const uint16_t *w, int cout, int cin, int k, int cout_p, int cin_p,
                         uint16_t *plane, void *stream);

/* ---------------------------------------------------------------------
 * 3x3 convolution, stride 1, zero padding 1, as an implicit GEMM
 * ([QI] module doc: every 3x3 conv an implicit GEMM, f16 inputs, f32
 * accumulation; `Rec::conv_s`; [VAE] `Conv2d::apply` for the definition):
 *   y[p][o] = oscale * sum_{tap,ci} plane[o][tap][ci] * x[src(p,tap)][ci]
 *             (+ bias[o] if bias != NULL)
 * where src(p,tap) is pixel (r+ky-1, c+kx-1) of the H x W image, zero
 * outside it. GEMM shape M = H*W, N = cout_p, K = 9*cin_p.
 *   x:     f16 NHWC [H*W][cin_p]        (cin_p: multiple of 64)
 *   w:     f16 3x3 plane from ig_pack_conv_weights, [cin_p/16][9][cout_p][16]
 *          (cout_p: multiple of 64)
 *   bias:  f32 [cout_p] or NULL
 *   y:     f32 NHWC [H*W][cout_p]
 * Limits (IG_EUNSUPPORTED past them), for every 3x3 entry point: the f16
 * input below 0x7fff0000 bytes (the kernels address it with 32-bit byte
 * offsets) and cin_p, cout_p <= 8192. The decoders check the same for
 * every conv input of their plan (a larger frame decodes in bands).
 * --------------------------------------------------------------------- */
int conv3x3_nhwc(const uint16_t *x, int H, int W, int cin_p, const uint16_t *w, int cout_p,
                 const float *bias, float oscale, float *y, void *stream);

/* ---------------------------------------------------------------------
 * 3x3 convolution of the nearest-2x upsampled image, the upsample folded
 * into the gather and never materialised ([QI] module doc; `Rec::conv_s`
 * with `up`; [VAE] `upsample2x` then `Conv2d::apply` for the definition).
 * x is the HALF-resolution H x W image; the output is 2H x 2W. Tap (ky,kx)
 * at output (r,c) reads x[(r+ky-1)/2][(c+kx-1)/2] when 0 <= r+ky-1 < 2H
 * and 0 <= c+kx-1 < 2W, else 0 (zero padding in upsampled coordinates).
 *   x: f16 [H*W][cin_p]; w: f16 3x3 plane (as conv3x3_nhwc); y: f32 [4*H*W][cout_p]
 * A guarded input ([QI] `guard`) is undone with oscale = 2^g.
 * --------------------------------------------------------------------- */
int conv3x3_up2_nhwc(const uint16_t *x, int H, int W, int cin_p, const uint16_t *w, int cout_p,
                     const float *bias, float oscale, float *y, void *stream);

/* The convolution family with one more output mode.
 *   mode 0: 1x1 conv ([QI] module doc: 1x1 convs as plain GEMMs),
 *           w = the 1x1 plane [cout_p][cin_p]; mode 1: 3x3 as conv3x3_nhwc;
 *   mode 2: 3x3 on the nearest-2x upsample as conv3x3_up2_nhwc.
 *   accumulate = 0: y = oscale*acc (+bias)
 *   accumulate = 1: y = y + oscale*acc (+bias)  -- the residual add of
 *                   [QI] `Rec::combine` mode 0 folded into the epilogue. */
int ig_conv_nhwc_ex(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w,
                    int cout_p, const float *bias, float oscale, int accumulate, float *y,
                    void *stream);

/* A 3x3 conv (mode 1) or folded-upsample 3x3 conv (mode 2) whose epilogue
 * also applies the next step of the pages' recipe ([QI] `Rec::resnet`:
 * h = conv1(xn), then xn = f16(RMS_norm(h + b1) -> SiLU); `output_rows`:
 * norm_out after the last up conv) -- RMSN_SRC on each output pixel:
 *   v = oscale*acc + bias; yn = f16(v * sqrt(c_real) / max(|v|_2, eps) * gamma),
 *   then SiLU (yn / (1 + e^-yn)) if silu,
 * so the f32 result need not be stored and re-read. Every channel of a
 * pixel must sit in one tile: cout_p must be 64 or 128 (IG_EUNSUPPORTED
 * otherwise); the pad channels' weights, bias and gamma must be zero.
 *   y: f32 [M][cout_p] receives v when non-NULL; yn: f16 [M][cout_p].
 * Other arguments and errors as ig_conv_nhwc_ex. */
int ig_conv3x3_norm_nhwc(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w, int cout_p,
                         int c_real, const float *bias, float oscale, const float *gamma, int silu, float eps,
                         float *y, uint16_t *yn, void *stream);

/* ---------------------------------------------------------------------
 * NT GEMM ([QI] `mmc`: B is the "plane" [N][K], A the activations [M][K];
 * the 1x1 convs and every attention product of [QI] `attention`):
 *   C[m][n] = oscale * sum_k A[m][k] * B[n][k] (+ bias[n])
 *   a: f16 [M][lda]; b: f16 [N][ldb]; c: [M][ldc], f32 or (c_is_f16) f16.
 * Requires K % 32 == 0, N % 64 == 0, lda/ldb multiples of 8, ldc >= N;
 * M is arbitrary (rows are masked).
 * --------------------------------------------------------------------- */
int gemm1x1(const uint16_t *a, int M, int K, int lda, const uint16_t *b, int N, int ldb,
            const float *bias, float oscale, void *c, int ldc, int c_is_f16, void *stream);

/* As gemm1x1 with the f32 output accumulated: C += oscale*A.B^T (+bias). */
int gemm1x1_acc(const uint16_t *a, int M, int K, int lda, const uint16_t *b, int N, int ldb,
                const float *bias, float oscale, float *c, int ldc, void *stream);

/* ---------------------------------------------------------------------
 * Per-pixel RMS_norm over the channels ([QI] RMSN_SRC, `Rec::rmsn`):
 *   v = x[p][:] + bias (bias on read, optional)
 *   y[p][c] = f16( v_c * sqrt(c_real) / max(||v||_2, eps) * gamma[c] )
 *   then, if silu, y <- y / (1 + e^-y) before the f16 store.
 * The sum runs over all cp channels (the pad holds zeros); sqrt uses
 * c_real, the real channel count.
 *   x: f32 [M][cp]; bias: f32 [cp] or NULL; gamma: f32 [cp], zero in pad;
 *   y: f16 [M][cp]. cp: multiple of 64, at most 1024. eps: 1e-12 on the
 *   pages.
 * --------------------------------------------------------------------- */
int rmsnorm_silu_f16(const float *x, int M, int cp, int c_real, const float *bias,
                     const float *gamma, int silu, float eps, uint16_t *y, void *stream);

/* A 3x3 conv (mode 1) or up conv (mode 2) whose epilogue also emits the
 * guarded f16 cast of its f32 result ([QI] `Rec::resnet` then
 * `run_blocks`: a stage's last resnet adds conv2 into the stream, which is
 * then cast, guarded, for the up conv):
 *   v = oscale * conv(x, w) + bias (+ y[p][o] if accumulate)
 *   y[p][o] = v (only if write_y);  yg[p][o] = f16( v * 2^-guard_log2 )
 * Shapes as ig_conv_nhwc_ex; y: f32 [M][cout_p] (read if accumulate);
 * yg: f16 [M][cout_p]. */
int ig_conv3x3_guard_out_nhwc(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w, int cout_p,
                              const float *bias, float oscale, int accumulate, float *y, int write_y, int guard_log2,
                              uint16_t *yg, void *stream);

/* The same norm and, from the same read of x, the guarded cast of the raw
 * stream ([QI] `Rec::resnet`: a resnet whose shortcut takes the stream
 * normalises it for conv1 and casts it, guarded, for the 1x1 shortcut):
 *   y as rmsnorm_silu_f16;  yg[p][c] = f16( (x[p][c] + bias[c]) * 2^-guard_log2 )
 * yg: f16 [M][cp]; guard_log2 in 0..14. Errors as rmsnorm_silu_f16. */
int rmsnorm_silu_guard_cast_f16(const float *x, int M, int cp, int c_real, const float *bias,
                                const float *gamma, int silu, float eps, uint16_t *y, int guard_log2,
                                uint16_t *yg, void *stream);

/* GroupNorm into the next conv's f16 input -- the norm of FLUX-class
 * decoders ([VAE] `GroupNorm::apply`; page "cortiq-engine 0.8.72,
 * src/gpu_wgpu/s2v_vae.rs", GN_PART_SRC / GN_FIN_SRC / GN_APPLY_SRC, `gn`):
 * the c_real real channels split into `groups` consecutive groups; per
 * group, over its channels and all M pixels of v = x + bias (bias optional),
 *   mean, var = mean((v - mean)^2),
 *   y = (v - mean) / sqrt(var + eps) * gamma + beta, then SiLU if silu,
 * stored as f16; pad channels (c_real <= c < cp) get 0.
 *   x: f32 [M][cp]; bias, gamma, beta: f32 [cp]; y: f16 [M][cp];
 *   ws: device workspace of ig_groupnorm_workspace_bytes(M, cp, groups)
 *   bytes (per-chunk statistics; contents on return are scratch).
 * cp must be a multiple of 4 up to 1024, groups 1..128 dividing c_real
 * (IG_EUNSUPPORTED otherwise); IG_EWORKSPACE when ws_bytes is short. */
size_t ig_groupnorm_workspace_bytes(int M, int cp, int groups);
int groupnorm_silu_f16(const float *x, int M, int cp, int c_real, int groups, const float *bias,
                       const float *gamma, const float *beta, int silu, float eps, void *ws, size_t ws_bytes,
                       uint16_t *y, void *stream);

/* groupnorm_silu_f16 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Its per-chunk statistics live in
 * a device array built into the library (about 1.5 MiB, one copy per GPU,
 * held until the process ends; every shape groupnorm_silu_f16 supports
 * fits, larger needs give IG_EUNSUPPORTED). Nothing is allocated: no
 * hipMalloc, no library allocator. The kernels write every scratch byte
 * they read, so no call depends on what an earlier one left there, but all
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * Arguments, outputs and errors otherwise as groupnorm_silu_f16 (IG_EHIP
 * if the array's device address cannot be obtained). */
int groupnorm_silu_f16_noalloc(const float *x, int M, int cp, int c_real, int groups, const float *bias,
                               const float *gamma, const float *beta, int silu, float eps, uint16_t *y,
                               void *stream);

/* GroupNorm with one read of its input: the producing 3x3 conv gathers the
 * group statistics in its epilogue, the norm merges them and applies
 * ([VAE] `GroupNorm::apply` for the definition; page "cortiq-engine
 * 0.8.72, src/gpu_wgpu/s2v_vae.rs", GN_PART_SRC, whose per-workgroup
 * partial sums here come from the conv's output tiles instead of a pass of
 * their own).
 *
 * ig_conv3x3_gn_stats_nhwc: ig_conv_nhwc_ex (mode 1 or 2, y written) that
 * also writes, for each 16 x 32-pixel tile pt of the output frame
 * (row-major; nchunk = ig_conv_gn_partials_bytes / (12 groups) of them) and each
 * group g of cpg = c_real / groups consecutive real channels, the tile's
 * (count, mean, M2 = sum of squared deviations) of the stored values
 * (after the accumulation, if any) as three floats at
 * part[(g * nchunk + pt) * 3]. The partials are f32, each tile's folded
 * four values at a time with Chan, Golub and LeVeque's update.
 *   part: f32, ig_conv_gn_partials_bytes(mode, H, W, groups) bytes.
 * cpg must be a multiple of 4 that divides 64 and cout_p a multiple of 64
 * (IG_EUNSUPPORTED otherwise); IG_EWORKSPACE when part_bytes is short.
 *
 * groupnorm_silu_f16_from_partials: groupnorm_silu_f16 of x (no bias on
 * read: the statistics are of x as stored) with the statistics merged, in
 * f64, from nchunk such partials per group (part [groups][nchunk][3]);
 * x is read once. ws: 16-byte-aligned device scratch of at least
 * 3 cp floats (per-channel offset, scale and shift). Errors as
 * groupnorm_silu_f16. */
size_t ig_conv_gn_partials_bytes(int mode, int H, int W, int groups);
int ig_conv3x3_gn_stats_nhwc(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w, int cout_p,
                             const float *bias, float oscale, int accumulate, float *y, int c_real, int groups,
                             float *part, size_t part_bytes, void *stream);
int groupnorm_silu_f16_from_partials(const float *x, int M, int cp, int c_real, int groups, const float *gamma,
                                     const float *beta, int silu, float eps, const float *part, int nchunk,
                                     void *ws, size_t ws_bytes, uint16_t *y, void *stream);

/* ---------------------------------------------------------------------
 * The range-guarded f16 cast of the raw residual stream ([QI] `guard`,
 * CAST_SRC, `Rec::cast`): y = f16((x + bias) * 2^-guard_log2); the
 * consuming conv multiplies 2^guard_log2 back in its f32 epilogue.
 *   x: f32 [M][C]; bias: f32 [C] or NULL; y: f16 [M][C];
 *   C % 4 == 0; guard_log2 in 0..14 (8 on the pages).
 * --------------------------------------------------------------------- */
int guard_cast(const float *x, int M, int C, const float *bias, int guard_log2, uint16_t *y,
               void *stream);

/* ---------------------------------------------------------------------
 * The residual combine ([QI] `Rec::combine`), f32 [M][C], with t = h + hb:
 *   mode 0 adds t into x; mode 1 sets x to t plus the shortcut s + sb;
 *   mode 2 sets x to t.
 *   hb, sb: [C] or NULL (zero). C % 4 == 0.
 * --------------------------------------------------------------------- */
int ig_combine(float *x, const float *h, const float *hb, const float *s, const float *sb, int M,
               int C, int mode, void *stream);

/* ---------------------------------------------------------------------
 * Row softmax of attention scores ([QI] `attention`: S f32 -> P f16;
 * [VAE] `AttnBlock::apply`: max-subtracted exp, divided by the row sum):
 *   P[r][j] = f16( exp(S[r][j] - max_r) / sum_{j<valid} exp(S[r][j] - max_r) )
 * for j < valid, and P[r][j] = 0 for valid <= j < ncols (padded keys).
 *   S: f32 [rows][lds]; P: f16 [rows][ldp]; ncols <= min(lds, ldp).
 * --------------------------------------------------------------------- */
int ig_softmax_rows_f16(const float *S, int rows, int lds, int valid, int ncols, uint16_t *P,
                        int ldp, void *stream);

/* ---------------------------------------------------------------------
 * The mid attention's core in one pass over the keys ([QI] `attention`:
 * S = q.k^T / sqrt(C), row softmax, O = P.V, V's bias after the product;
 * [VAE] `AttnBlock::apply`: max-subtracted softmax):
 *   out[i][c] = f16( sum_{j<m} softmax_j(q_i . k_j / sqrt(C)) vt[c][j] + bv[c] )
 * The softmax is taken online over blocks of 32 keys (a running sum per
 * query); no score or probability matrix is stored. Each block's weights
 * exp(s - ref) are rounded to f16 against a per-query reference ref fixed
 * for the pass (the first block's max; a later block more than 2^15 above
 * it makes the kernel redo the pass with the true max), and divided by
 * their sum at the end (the chunked path rounds the normalised
 * probabilities instead), so the two agree to f16 rounding, not bit for
 * bit.
 *   q, k: f16 [ld][C] row-major; rows m..ld-1 are read, never used.
 *   vt:   f16 V^T [C][ld].
 *   bv:   f32 [C] or NULL.      out: f16 [m][C].
 *   ws:   device scratch of ws_bytes >= ig_attention_workspace_bytes(m, C)
 *         (0 bytes for small m: ws may then be NULL); its contents on
 *         entry do not matter.
 * C must be 128, 256, 384 or 512 (IG_EUNSUPPORTED otherwise: other
 * widths take the chunked path of decoder_forward); ld >= m rounded up to 32,
 * ld % 8 == 0 and ld * C * 2 < 0x7fff0000 (the kernel addresses q, k and
 * V^T with 32-bit byte offsets); q, k, vt, out 16-byte aligned. m < 2^22.
 * --------------------------------------------------------------------- */
size_t ig_attention_workspace_bytes(int m, int C);
int attention_f16(const uint16_t *q, const uint16_t *k, const uint16_t *vt, int m, int ld, int C,
                  const float *bv, void *ws, size_t ws_bytes, uint16_t *out, void *stream);

/* Latent ingest ([QI] `decode`: the NCHW latent becomes an NHWC f16 conv
 * input): y[p][c] = f16(z[c][p]) for c < zc, 0 for zc <= c < cp.
 *   z: f32 [zc][M]; y: f16 [M][cp]. */
int ig_latent_to_nhwc_f16(const float *z, int zc, int M, int cp, uint16_t *y, void *stream);

/* Output stage ([QI] OUT_SRC): out[ch][p] = y[p][ch] (+ bias[ch]) for
 * ch < nch. y: f32 [M][ld]; bias: [nch] or NULL; out: f32 [nch][M]. */
int ig_nhwc_to_nchw(const float *y, int M, int ld, int nch, const float *bias, float *out,
                    void *stream);

/* The decoder's output convolution ([QI] `output_rows` and OUT_SRC; [VAE]
 * `Conv2d::apply`): a 3x3 conv (stride 1, zero padding 1) with few output
 * channels, written into the NCHW frame with the bias,
 *   out[o][y*W + x] = b[o] + sum_{ky,kx,c} w[o][c][ky][kx] x[(y+ky-1)*W + x+kx-1][c]
 * for o < cout.
 *   x: f16 NHWC [H*W][cin_p], cin_p a multiple of 64, 16-byte aligned;
 *   w: the blocked 3x3 plane of ig_pack_conv_weights (cout_p >= cout);
 *   bias: f32 [cout] or NULL; out: f32 [cout][H*W].
 * cout must be 1..16 (IG_EUNSUPPORTED otherwise). */
int ig_conv3x3_out_nchw(const uint16_t *x, int H, int W, int cin_p, const uint16_t *w, int cout, int cout_p,
                        const float *bias, float *out, void *stream);

/* The DupUp shortcut ([QI] DUPUP_SRC and `run_blocks`): the half-resolution
 * input, its channels repeated and moved to space, added onto the 2x grid.
 * Output pixel (2y + sy, 2x + sx), channel o < cout, gets src pixel (y, x)'s
 * channel (o * factor + 4 * (ft - 1) + 2 * sy + sx) / repeats. With
 * factor = repeats = 4 and ft = 1 every output channel reads its own
 * channel: the nearest-2x upsample of src added into x (in = out channels).
 *   src: f32 [H*W][cin_p]; x: f32 [4*H*W][cout_p], 16-byte aligned,
 *   cout_p % 4 == 0; every shuffled channel index must be < cin_p. */
int ig_dupup_add(const float *src, int H, int W, int cin_p, float *x, int cout, int cout_p,
                 int factor, int repeats, int ft, void *stream);

/* Zero rows [r0, r1) of an f16 matrix with row length ld (a fill kernel,
 * safe under stream capture). */
int ig_zero_rows_f16(uint16_t *y, int r0, int r1, int ld, void *stream);

/* ---------------------------------------------------------------------
 * The whole decoder on one stream ([QI] `decode`, `Rec::resnet`,
 * `attention`, `run_blocks`, `output_rows`; [VAE] `VaeDecoder::decode`):
 *   f16(latent) -> conv_in -> resnet -> attention -> resnet
 *   -> per up stage: resnets, x = 2^g conv_up2(f16(x 2^-g)) + b
 *      (+ the DupUp shuffle of the stage's input when dupup)
 *   -> f16(RMS_norm(x; norm_out) -> SiLU) -> conv_out -> NCHW output.
 * Every weight is device memory the caller owns, packed by
 * ig_pack_conv_weights; biases and gammas are f32 zero-padded to the
 * padded widths. All widths are padded to multiples of 64.
 * --------------------------------------------------------------------- */
typedef struct ig_conv_w {
    const uint16_t *w; /* plane from ig_pack_conv_weights (layout by k) */
    const float *b;    /* [cout_p], or NULL for no bias */
    int cin, cout;     /* real channel counts */
    int cin_p, cout_p; /* padded widths */
    int k;             /* 1 or 3 */
} ig_conv_w;

typedef struct ig_resnet_w {
    const float *g1; /* [cin_p] gamma of the first RMS_norm */
    ig_conv_w c1;    /* 3x3 cin -> cout */
    const float *g2; /* [cout_p] gamma of the second RMS_norm */
    ig_conv_w c2;    /* 3x3 cout -> cout */
    int has_sc;      /* 1: a 1x1 shortcut cin -> cout (guarded input) */
    ig_conv_w sc;
    const float *beta1, *beta2; /* [cin_p], [cout_p]: GroupNorm's beta (IG_NORM_GROUP only) */
} ig_resnet_w;

typedef struct ig_attn_w {
    const float *gamma;      /* [c] RMS_norm gamma (no SiLU) */
    ig_conv_w q, k, v, proj; /* 1x1 c -> c; c % 64 == 0, unpadded */
    const float *beta;       /* [c] GroupNorm's beta (IG_NORM_GROUP only) */
} ig_attn_w;

typedef struct ig_up_w {
    int n_res;
    ig_resnet_w res[IG_MAX_RES];
    int has_up;   /* 1: a nearest-2x upsample conv ends the stage */
    ig_conv_w up; /* 3x3 */
    /* 1 (with has_up): after the up conv, add the DupUp shortcut of the
     * stage's input ([QI] `run_blocks`, DUPUP_SRC; ig_dupup_add) with
     * factor = 4 dupup_ft and repeats = up.cout * factor / cin, cin the
     * stage input's real channels (up.cout * factor must be a multiple of
     * it). dupup_ft: the temporal factor, 1 for images. */
    int dupup, dupup_ft;
} ig_up_w;

typedef struct ig_decoder {
    int zc;            /* latent channels */
    ig_conv_w conv_in; /* 3x3 zc -> c */
    ig_resnet_w mid[2];
    ig_attn_w attn;
    int n_up;
    ig_up_w ups[IG_MAX_UP];
    const float *norm_out_gamma; /* [cp] */
    int norm_out_c;              /* real channels of norm_out */
    ig_conv_w conv_out;          /* 3x3 c -> out channels (<= 64) */
    /* The norm of every norm site (the resnets' two, the attention's,
     * norm_out): IG_NORM_RMS (0; eps 1e-12; betas unused) or IG_NORM_GROUP
     * (a FLUX-class decoder, [VAE] `VaeDecoder::decode`: GroupNorm over
     * norm_groups groups of the real channels, eps norm_eps, with the
     * betas; each site's real width a multiple of norm_groups, padded
     * width <= 1024, groups <= 128). GroupNorm's statistics span the frame,
     * so a GroupNorm decoder does not run in bands (IG_EUNSUPPORTED). */
    int norm_kind, norm_groups;
    float norm_eps;
    const float *norm_out_beta; /* [cp] */
} ig_decoder;

/* Workspace bytes decoder_forward needs for an h0 x w0 latent. q_chunk
 * selects the attention: q_chunk <= 0 takes the single-pass kernel of
 * attention_f16 when the attention width is 128, 256, 384 or 512 (else query chunks of
 * 16384 rows); q_chunk > 0 takes the chunked path (scores' row statistics,
 * then P, then P.V) over chunks of q_chunk query rows. Returns 0
 * if the descriptor or the sizes are invalid (see ig_last_error()). */
size_t ig_decoder_workspace_bytes(const ig_decoder *dec, int h0, int w0, int q_chunk);

/* Decode one latent. latent: f32 NCHW [zc][h0*w0]; out: f32 NCHW
 * [conv_out.cout][H*W] with H = h0 * 2^(stages with has_up), likewise W.
 * guard_log2 in 0..14; ws: device workspace of ws_bytes >=
 * ig_decoder_workspace_bytes(). On a validation error nothing is
 * enqueued and out is untouched. */
int decoder_forward(const ig_decoder *dec, const float *latent, int h0, int w0, int guard_log2,
                    int q_chunk, void *ws, size_t ws_bytes, float *out, void *stream);

/* ---------------------------------------------------------------------
 * Banded decode ([QI] the bands section, `run_blocks`, `output_rows`).
 * After the mid block every step only looks at nearby pixels, so up blocks
 * band_from.. can run on horizontal bands of band_rows kept output rows.
 * Each band starts from the rows of the whole-frame stream (saved at block
 * band_from's input) that its kept rows depend on: tracing back, a 3x3 conv
 * widens the range by a row per side and an upsample halves it, rounded
 * outward, both cut at the frame's edges. Rows near a band's edge see zero
 * padding where the whole frame has data, and so differ, but no kept row
 * depends on them: the kept rows equal the whole-frame decode's exactly.
 * The workspace holds the whole-frame tensors up to block band_from and one
 * band's tensors after it.
 * band_rows <= 0 or band_from >= n_up: the whole frame (decoder_forward).
 * Returns 0 from the size query on invalid arguments (ig_last_error()).
 * --------------------------------------------------------------------- */
size_t ig_decoder_bands_workspace_bytes(const ig_decoder *dec, int h0, int w0, int q_chunk, int band_rows,
                                        int band_from);
int decoder_forward_bands(const ig_decoder *dec, const float *latent, int h0, int w0, int guard_log2,
                          int q_chunk, int band_rows, int band_from, void *ws, size_t ws_bytes, float *out,
                          void *stream);

/* The band planner alone (host only, no device work): for a decoder of
 * n_up up blocks (block i: n_res[i] resnets of two 3x3 convs, then, if
 * has_up[i], a nearest-2x upsample and a 3x3 conv) followed by a 3x3
 * conv_out, latent height h0, and kept output rows [keep_lo, keep_hi):
 * input[0..1] = the rows [lo, hi) of block band_from's input the band
 * starts from; feed[2i..2i+1] = the rows block i (>= band_from, with
 * has_up) feeds to its upsample, (0, 0) otherwise. feed: [2 * n_up]. */
int ig_band_plan(int n_up, const int *n_res, const int *has_up, int h0, int band_from, int keep_lo,
                 int keep_hi, int *input, int *feed);

/* Measurement hook, for benchmarks (not a step of the method): while
 * dev_buf is set, every launch of the 3x3 conv kernel that holds its
 * weights in registers (cin_p = cout_p = 128) has its first wave write,
 * into dev_buf (device memory, 4 x uint64, owned by the caller), the
 * shader-clock counter and the 100 MHz real-time counter at the wave's
 * start and at its end: [clk0, rt0, clk1, rt1]. The clock the kernel ran
 * at is (clk1 - clk0) / ((rt1 - rt0) / 1e8) Hz. NULL stops it. The
 * setting is process-wide and the buffer is rewritten by each launch:
 * not for concurrent launches. Returns 0. */
int ig_set_clock_probe(void *dev_buf);

#ifdef __cplusplus
}
#endif

#endif /* IG_CONV_H */
