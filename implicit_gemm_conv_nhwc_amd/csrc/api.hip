// The C entry points of libigconv (declared in include/ig_conv.h): argument
// validation, then the launch. Validation happens before anything is
// enqueued, so a rejected call leaves every output untouched (the
// "declined, output untouched" contract of the page "cortiq-engine 0.8.3,
// src/gpu_wgpu/qi21_vae.rs", `decode` and `decline`).
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "ig_internal.h"

namespace ig {

static thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

int check_launch(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(IG_EHIP, "%s: %s", what, hipGetErrorString(e));
    return IG_OK;
}

static int check_ptr(const void *p, const char *name, bool need16 = true)
{
    if (!p) return fail(IG_EINVAL, "%s is NULL", name);
    if (need16 && !aligned16(p)) return fail(IG_EINVAL, "%s is not 16-byte aligned", name);
    return IG_OK;
}

// Shapes common to the convolutions (mode 0: 1x1, 1: 3x3, 2: 3x3 up2).
static int check_conv(const void *x, int H, int W, int cin_p, const void *w, int cout_p,
                      const float *bias, const void *y, int mode, bool *empty)
{
    *empty = false;
    if (mode < 0 || mode > 2) return fail(IG_EINVAL, "conv mode %d is not 0, 1 or 2", mode);
    if (H < 0 || W < 0) return fail(IG_EINVAL, "negative image size %dx%d", H, W);
    if (cin_p <= 0 || cin_p % 64) return fail(IG_EUNSUPPORTED, "cin_p=%d is not a positive multiple of 64", cin_p);
    if (cout_p <= 0 || cout_p % 64) return fail(IG_EUNSUPPORTED, "cout_p=%d is not a positive multiple of 64", cout_p);
    if (cin_p > kConvMaxChannels || cout_p > kConvMaxChannels)
        return fail(IG_EUNSUPPORTED, "cin_p=%d / cout_p=%d exceed %d", cin_p, cout_p, kConvMaxChannels);
    const int64_t mout = (int64_t)H * W * (mode == 2 ? 4 : 1);
    if ((int64_t)H * W * cin_p >= (1LL << 31) || mout * cout_p >= (1LL << 40) || mout >= (1LL << 31) ||
        (mode != 0 && (int64_t)H * W * cin_p * 2 >= kConvInMaxBytes))
        return fail(IG_EUNSUPPORTED, "image %dx%d with %d/%d channels is too large", H, W, cin_p, cout_p);
    if (H == 0 || W == 0) {
        *empty = true;
        return IG_OK;
    }
    int r;
    if ((r = check_ptr(x, "x")) || (r = check_ptr(w, "w")) || (r = check_ptr(y, "y"))) return r;
    if (bias && ((uintptr_t)bias & 3)) return fail(IG_EINVAL, "bias is not 4-byte aligned");
    return IG_OK;
}

static int conv_any(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w,
                    int cout_p, const float *bias, float oscale, int accumulate, float *y,
                    void *stream)
{
    clear_error();
    bool empty;
    int r = check_conv(x, H, W, cin_p, w, cout_p, bias, y, mode, &empty);
    if (r || empty) return r;
    IgemmArgs a{};
    a.a = reinterpret_cast<const _Float16 *>(x);
    a.b = reinterpret_cast<const _Float16 *>(w);
    a.bias = bias;
    a.c = y;
    a.M = H * W * (mode == 2 ? 4 : 1);
    a.N = cout_p;
    a.K = (mode == 0 ? 1 : 9) * cin_p;
    a.lda = cin_p;
    a.ldb = a.K;
    a.ldc = cout_p;
    a.H = H;
    a.W = W;
    a.cin_p = cin_p;
    a.oscale = oscale;
    a.accumulate = accumulate ? 1 : 0;
    a.out_f16 = 0;
    (void)hipGetLastError();
    launch_igemm(mode == 0 ? kGemm : (mode == 1 ? kConv3x3 : kConv3x3Up2), a,
                 reinterpret_cast<hipStream_t>(stream));
    return check_launch("conv launch");
}

static int gemm_any(const uint16_t *a, int M, int K, int lda, const uint16_t *b, int N, int ldb,
                    const float *bias, float oscale, void *c, int ldc, int c_is_f16,
                    int accumulate, void *stream)
{
    clear_error();
    if (M < 0 || K <= 0 || N <= 0) return fail(IG_EINVAL, "bad GEMM size M=%d N=%d K=%d", M, N, K);
    if (K % 32) return fail(IG_EUNSUPPORTED, "K=%d is not a multiple of 32", K);
    if (N % 64) return fail(IG_EUNSUPPORTED, "N=%d is not a multiple of 64", N);
    if (lda < K || ldb < K || ldc < N) return fail(IG_EINVAL, "leading dimensions too small");
    if (lda % 8 || ldb % 8) return fail(IG_EUNSUPPORTED, "lda/ldb must be multiples of 8");
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(a, "a")) || (r = check_ptr(b, "b")) || (r = check_ptr(c, "c", false))) return r;
    if (((uintptr_t)c & (c_is_f16 ? 1 : 3))) return fail(IG_EINVAL, "c is misaligned");
    if (bias && ((uintptr_t)bias & 3)) return fail(IG_EINVAL, "bias is not 4-byte aligned");
    if (c_is_f16 && accumulate) return fail(IG_EUNSUPPORTED, "f16 output cannot accumulate");
    IgemmArgs g{};
    g.a = reinterpret_cast<const _Float16 *>(a);
    g.b = reinterpret_cast<const _Float16 *>(b);
    g.bias = bias;
    g.c = c;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.oscale = oscale;
    g.accumulate = accumulate;
    g.out_f16 = c_is_f16 ? 1 : 0;
    (void)hipGetLastError();
    launch_igemm(kGemm, g, reinterpret_cast<hipStream_t>(stream));
    return check_launch("gemm launch");
}

// GroupNorm's checks shared by both entry points; IG_OK, or the status
int groupnorm_check(const float *x, int M, int cp, int c_real, int groups, const float *bias, const float *gamma,
                    const float *beta, float eps, uint16_t *y)
{
    if (M < 0) return fail(IG_EINVAL, "M=%d is negative", M);
    if (cp <= 0 || c_real <= 0 || c_real > cp || groups <= 0) return fail(IG_EINVAL, "bad channels cp=%d c_real=%d groups=%d", cp, c_real, groups);
    if (!gn_supported(cp, c_real, groups))
        return fail(IG_EUNSUPPORTED, "GroupNorm needs cp %% 4 == 0 (<= 1024) and 1..128 groups dividing c_real");
    if (!(eps > 0.f)) return fail(IG_EINVAL, "eps must be positive");
    if ((int64_t)M * cp >= (1LL << 40)) return fail(IG_EUNSUPPORTED, "too many elements");
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(x, "x")) || (r = check_ptr(gamma, "gamma")) || (r = check_ptr(beta, "beta")) ||
        (r = check_ptr(y, "y", false)))
        return r;
    if (bias && (r = check_ptr(bias, "bias"))) return r;
    return IG_OK;
}


}  // namespace ig

using namespace ig;

extern "C" {

const char *ig_last_error(void) { return g_err; }

int ig_version(void) { return (1 << 16) | 0; }

int ig_set_clock_probe(void *dev_buf)
{
    ig::set_clock_probe(dev_buf);
    return 0;
}

int ig_pack_conv_weights(const uint16_t *w, int cout, int cin, int k, int cout_p, int cin_p,
                         uint16_t *plane, void *stream)
{
    clear_error();
    if (k != 1 && k != 3) return fail(IG_EUNSUPPORTED, "k=%d is not 1 or 3", k);
    if (cout <= 0 || cin <= 0 || cout_p < cout || cin_p < cin)
        return fail(IG_EINVAL, "bad channel counts cout=%d/%d cin=%d/%d", cout, cout_p, cin, cin_p);
    if (cout_p % 64 || cin_p % 64) return fail(IG_EUNSUPPORTED, "padded widths must be multiples of 64");
    if (!w || !plane) return fail(IG_EINVAL, "NULL weight pointer");
    if (((uintptr_t)w & 1) || ((uintptr_t)plane & 1)) return fail(IG_EINVAL, "misaligned f16 pointer");
    (void)hipGetLastError();
    launch_pack_weights(reinterpret_cast<const _Float16 *>(w), cout, cin, k, cout_p, cin_p,
                        reinterpret_cast<_Float16 *>(plane), reinterpret_cast<hipStream_t>(stream));
    return check_launch("pack launch");
}

int conv3x3_nhwc(const uint16_t *x, int H, int W, int cin_p, const uint16_t *w, int cout_p,
                 const float *bias, float oscale, float *y, void *stream)
{
    return conv_any(x, H, W, cin_p, 1, w, cout_p, bias, oscale, 0, y, stream);
}

int conv3x3_up2_nhwc(const uint16_t *x, int H, int W, int cin_p, const uint16_t *w, int cout_p,
                     const float *bias, float oscale, float *y, void *stream)
{
    return conv_any(x, H, W, cin_p, 2, w, cout_p, bias, oscale, 0, y, stream);
}

int ig_conv_nhwc_ex(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w,
                    int cout_p, const float *bias, float oscale, int accumulate, float *y,
                    void *stream)
{
    return conv_any(x, H, W, cin_p, mode, w, cout_p, bias, oscale, accumulate, y, stream);
}

int ig_conv3x3_guard_out_nhwc(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w, int cout_p,
                              const float *bias, float oscale, int accumulate, float *y, int write_y, int guard_log2,
                              uint16_t *yg, void *stream)
{
    clear_error();
    if (mode != 1 && mode != 2) return fail(IG_EINVAL, "mode %d is not a 3x3 mode", mode);
    if (guard_log2 < 0 || guard_log2 > 14) return fail(IG_EINVAL, "guard_log2=%d outside 0..14", guard_log2);
    if ((accumulate || write_y) && !y) return fail(IG_EINVAL, "y is NULL but read or written");
    bool empty;
    int r = check_conv(x, H, W, cin_p, w, cout_p, bias, yg, mode, &empty);
    if (r || empty) return r;
    if (y && (r = check_ptr(y, "y"))) return r;
    IgemmArgs a{};
    a.a = reinterpret_cast<const _Float16 *>(x);
    a.b = reinterpret_cast<const _Float16 *>(w);
    a.bias = bias;
    a.c = y;
    a.M = H * W * (mode == 2 ? 4 : 1);
    a.N = cout_p;
    a.K = 9 * cin_p;
    a.lda = cin_p;
    a.ldb = a.K;
    a.ldc = cout_p;
    a.H = H;
    a.W = W;
    a.cin_p = cin_p;
    a.oscale = oscale;
    a.accumulate = accumulate ? 1 : 0;
    a.write_out = write_y ? 1 : 0;
    a.yg = reinterpret_cast<_Float16 *>(yg);
    a.gscale = ldexpf(1.f, -guard_log2);
    (void)hipGetLastError();
    launch_conv_halo(mode == 1 ? kConv3x3 : kConv3x3Up2, a, reinterpret_cast<hipStream_t>(stream));
    return check_launch("conv+cast launch");
}

int ig_conv3x3_norm_nhwc(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w, int cout_p,
                         int c_real, const float *bias, float oscale, const float *gamma, int silu, float eps,
                         float *y, uint16_t *yn, void *stream)
{
    clear_error();
    if (mode != 1 && mode != 2) return fail(IG_EINVAL, "mode %d is not a 3x3 mode", mode);
    if (cout_p != 64 && cout_p != 128)
        return fail(IG_EUNSUPPORTED, "the fused norm needs cout_p 64 or 128, got %d", cout_p);
    if (c_real <= 0 || c_real > cout_p) return fail(IG_EINVAL, "c_real=%d outside 1..cout_p", c_real);
    if (!(eps > 0.f)) return fail(IG_EINVAL, "eps must be positive");
    bool empty;
    int r = check_conv(x, H, W, cin_p, w, cout_p, bias, y ? y : reinterpret_cast<float *>(yn), mode, &empty);
    if (r || empty) return r;
    if ((r = check_ptr(gamma, "gamma")) || (r = check_ptr(yn, "yn"))) return r;
    IgemmArgs a{};
    a.a = reinterpret_cast<const _Float16 *>(x);
    a.b = reinterpret_cast<const _Float16 *>(w);
    a.bias = bias;
    a.c = y;
    a.M = H * W * (mode == 2 ? 4 : 1);
    a.N = cout_p;
    a.K = 9 * cin_p;
    a.lda = cin_p;
    a.ldb = a.K;
    a.ldc = cout_p;
    a.H = H;
    a.W = W;
    a.cin_p = cin_p;
    a.oscale = oscale;
    a.ngamma = gamma;
    a.ny = reinterpret_cast<_Float16 *>(yn);
    a.norm_c = c_real;
    a.norm_silu = silu ? 1 : 0;
    a.norm_eps = eps;
    a.write_out = y ? 1 : 0;
    (void)hipGetLastError();
    launch_conv_halo(mode == 1 ? kConv3x3 : kConv3x3Up2, a, reinterpret_cast<hipStream_t>(stream));
    return check_launch("conv+norm launch");
}

size_t ig_conv_gn_partials_bytes(int mode, int H, int W, int groups)
{
    if ((mode != 1 && mode != 2) || H < 0 || W < 0 || groups <= 0) return 0;
    return (size_t)groups * conv_gn_chunks(mode == 1 ? kConv3x3 : kConv3x3Up2, H, W) * 3 * sizeof(float);
}

int ig_conv3x3_gn_stats_nhwc(const uint16_t *x, int H, int W, int cin_p, int mode, const uint16_t *w, int cout_p,
                             const float *bias, float oscale, int accumulate, float *y, int c_real, int groups,
                             float *part, size_t part_bytes, void *stream)
{
    clear_error();
    if (mode != 1 && mode != 2) return fail(IG_EINVAL, "mode %d is not a 3x3 mode", mode);
    if (!conv_gn_stats_supported(cout_p, c_real, groups))
        return fail(IG_EUNSUPPORTED, "GroupNorm(%d) statistics over %d of %d channels: groups of 4..64 channels "
                                     "dividing 64 only", groups, c_real, cout_p);
    bool empty;
    int r = check_conv(x, H, W, cin_p, w, cout_p, bias, y, mode, &empty);
    if (r || empty) return r;
    const size_t need = ig_conv_gn_partials_bytes(mode, H, W, groups);
    if (!part || part_bytes < need)
        return fail(IG_EWORKSPACE, "GroupNorm partials of %zu bytes, %zu needed", part_bytes, need);
    if ((r = check_ptr(part, "part"))) return r;
    IgemmArgs a{};
    a.a = reinterpret_cast<const _Float16 *>(x);
    a.b = reinterpret_cast<const _Float16 *>(w);
    a.bias = bias;
    a.c = y;
    a.M = H * W * (mode == 2 ? 4 : 1);
    a.N = cout_p;
    a.K = 9 * cin_p;
    a.lda = cin_p;
    a.ldb = a.K;
    a.ldc = cout_p;
    a.H = H;
    a.W = W;
    a.cin_p = cin_p;
    a.oscale = oscale;
    a.accumulate = accumulate ? 1 : 0;
    a.gn_part = part;
    a.gn_cpg = c_real / groups;
    a.gn_creal = c_real;
    a.gn_nchunk = conv_gn_chunks(mode == 1 ? kConv3x3 : kConv3x3Up2, H, W);
    (void)hipGetLastError();
    launch_conv_halo(mode == 1 ? kConv3x3 : kConv3x3Up2, a, reinterpret_cast<hipStream_t>(stream));
    return check_launch("conv+GroupNorm statistics launch");
}

int groupnorm_silu_f16_from_partials(const float *x, int M, int cp, int c_real, int groups, const float *gamma,
                                     const float *beta, int silu, float eps, const float *part, int nchunk,
                                     void *ws, size_t ws_bytes, uint16_t *y, void *stream)
{
    clear_error();
    int r = groupnorm_check(x, M, cp, c_real, groups, nullptr, gamma, beta, eps, y);
    if (r || M == 0) return r;
    if (nchunk <= 0) return fail(IG_EINVAL, "nchunk=%d", nchunk);
    if ((r = check_ptr(part, "part"))) return r;
    if (!ws || ((uintptr_t)ws & 15) || ws_bytes < (size_t)cp * 3 * sizeof(float))
        return fail(IG_EWORKSPACE, "GroupNorm table of %zu bytes (16-byte aligned), %zu needed", ws_bytes,
                    (size_t)cp * 3 * sizeof(float));
    (void)hipGetLastError();
    launch_groupnorm_partials(x, M, cp, c_real, groups, gamma, beta, silu, eps, part, nchunk,
                              static_cast<float *>(ws), reinterpret_cast<_Float16 *>(y),
                              reinterpret_cast<hipStream_t>(stream));
    return check_launch("groupnorm (partials) launch");
}

int gemm1x1(const uint16_t *a, int M, int K, int lda, const uint16_t *b, int N, int ldb,
            const float *bias, float oscale, void *c, int ldc, int c_is_f16, void *stream)
{
    return gemm_any(a, M, K, lda, b, N, ldb, bias, oscale, c, ldc, c_is_f16, 0, stream);
}

int gemm1x1_acc(const uint16_t *a, int M, int K, int lda, const uint16_t *b, int N, int ldb,
                const float *bias, float oscale, float *c, int ldc, void *stream)
{
    return gemm_any(a, M, K, lda, b, N, ldb, bias, oscale, c, ldc, 0, 1, stream);
}

static int rmsnorm_any(const float *x, int M, int cp, int c_real, const float *bias, const float *gamma, int silu,
                       float eps, uint16_t *y, int guard_log2, uint16_t *yg, void *stream)
{
    clear_error();
    if (yg && (guard_log2 < 0 || guard_log2 > 14)) return fail(IG_EINVAL, "guard_log2=%d outside 0..14", guard_log2);
    if (M < 0) return fail(IG_EINVAL, "M=%d is negative", M);
    if (cp <= 0 || cp % 64 || cp > 1024) return fail(IG_EUNSUPPORTED, "cp=%d is not a multiple of 64 in 64..1024", cp);
    if (c_real <= 0 || c_real > cp) return fail(IG_EINVAL, "c_real=%d outside 1..cp", c_real);
    if (!(eps > 0.f)) return fail(IG_EINVAL, "eps must be positive");
    if ((int64_t)M * cp >= (1LL << 40)) return fail(IG_EUNSUPPORTED, "too many elements");
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(x, "x")) || (r = check_ptr(gamma, "gamma")) || (r = check_ptr(y, "y"))) return r;
    if (bias && (r = check_ptr(bias, "bias"))) return r;
    if (yg && (r = check_ptr(yg, "yg"))) return r;
    (void)hipGetLastError();
    launch_rmsnorm(x, M, cp, c_real, bias, gamma, silu, eps, reinterpret_cast<_Float16 *>(y),
                   reinterpret_cast<hipStream_t>(stream), reinterpret_cast<_Float16 *>(yg), guard_log2);
    return check_launch("rmsnorm launch");
}

int rmsnorm_silu_f16(const float *x, int M, int cp, int c_real, const float *bias,
                     const float *gamma, int silu, float eps, uint16_t *y, void *stream)
{
    return rmsnorm_any(x, M, cp, c_real, bias, gamma, silu, eps, y, 0, nullptr, stream);
}

int rmsnorm_silu_guard_cast_f16(const float *x, int M, int cp, int c_real, const float *bias,
                                const float *gamma, int silu, float eps, uint16_t *y, int guard_log2,
                                uint16_t *yg, void *stream)
{
    if (!yg) {
        clear_error();
        return fail(IG_EINVAL, "yg is NULL");
    }
    return rmsnorm_any(x, M, cp, c_real, bias, gamma, silu, eps, y, guard_log2, yg, stream);
}

size_t ig_groupnorm_workspace_bytes(int M, int cp, int groups)
{
    if (M < 0 || cp <= 0 || groups <= 0) return 0;
    return gn_workspace_bytes(M, cp, groups);
}

int groupnorm_silu_f16_noalloc(const float *x, int M, int cp, int c_real, int groups, const float *bias,
                               const float *gamma, const float *beta, int silu, float eps, uint16_t *y, void *stream)
{
    clear_error();
    int r = groupnorm_check(x, M, cp, c_real, groups, bias, gamma, beta, eps, y);
    if (r || M == 0) return r;
    const size_t need = gn_workspace_bytes(M, cp, groups);
    if (need > gn_scratch_bytes())
        return fail(IG_EUNSUPPORTED, "GroupNorm needs %zu bytes of scratch, the built-in array holds %zu", need,
                    gn_scratch_bytes());
    void *ws = gn_scratch_ptr();
    if (!ws) return fail(IG_EHIP, "the GroupNorm scratch array's device address is not available");
    (void)hipGetLastError();
    launch_groupnorm(x, M, cp, c_real, groups, bias, gamma, beta, silu, eps, ws, reinterpret_cast<_Float16 *>(y),
                     reinterpret_cast<hipStream_t>(stream));
    return check_launch("groupnorm launch");
}

int groupnorm_silu_f16(const float *x, int M, int cp, int c_real, int groups, const float *bias,
                       const float *gamma, const float *beta, int silu, float eps, void *ws, size_t ws_bytes,
                       uint16_t *y, void *stream)
{
    clear_error();
    int r = groupnorm_check(x, M, cp, c_real, groups, bias, gamma, beta, eps, y);
    if (r || M == 0) return r;
    if (!ws || ws_bytes < gn_workspace_bytes(M, cp, groups))
        return fail(IG_EWORKSPACE, "GroupNorm workspace of %zu bytes, %zu needed", ws_bytes,
                    gn_workspace_bytes(M, cp, groups));
    (void)hipGetLastError();
    launch_groupnorm(x, M, cp, c_real, groups, bias, gamma, beta, silu, eps, ws, reinterpret_cast<_Float16 *>(y),
                     reinterpret_cast<hipStream_t>(stream));
    return check_launch("groupnorm launch");
}

int guard_cast(const float *x, int M, int C, const float *bias, int guard_log2, uint16_t *y,
               void *stream)
{
    clear_error();
    if (M < 0 || C <= 0) return fail(IG_EINVAL, "bad size M=%d C=%d", M, C);
    if (C % 4) return fail(IG_EUNSUPPORTED, "C=%d is not a multiple of 4", C);
    if (guard_log2 < 0 || guard_log2 > 14) return fail(IG_EINVAL, "guard_log2=%d outside 0..14", guard_log2);
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(x, "x")) || (r = check_ptr(y, "y", false))) return r;
    if ((uintptr_t)y & 7) return fail(IG_EINVAL, "y is not 8-byte aligned");
    if (bias && (r = check_ptr(bias, "bias"))) return r;
    (void)hipGetLastError();
    launch_guard_cast(x, M, C, bias, guard_log2, reinterpret_cast<_Float16 *>(y),
                      reinterpret_cast<hipStream_t>(stream));
    return check_launch("guard_cast launch");
}

int ig_combine(float *x, const float *h, const float *hb, const float *s, const float *sb, int M,
               int C, int mode, void *stream)
{
    clear_error();
    if (M < 0 || C <= 0 || C % 4) return fail(IG_EINVAL, "bad size M=%d C=%d (C %% 4 == 0)", M, C);
    if (mode < 0 || mode > 2) return fail(IG_EINVAL, "mode %d is not 0, 1 or 2", mode);
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(x, "x")) || (r = check_ptr(h, "h"))) return r;
    if (mode == 1 && (r = check_ptr(s, "s"))) return r;
    if (hb && (r = check_ptr(hb, "hb"))) return r;
    if (sb && (r = check_ptr(sb, "sb"))) return r;
    (void)hipGetLastError();
    launch_combine(x, h, hb, s, sb, M, C, mode, reinterpret_cast<hipStream_t>(stream));
    return check_launch("combine launch");
}

int ig_softmax_rows_f16(const float *S, int rows, int lds, int valid, int ncols, uint16_t *P,
                        int ldp, void *stream)
{
    clear_error();
    if (rows < 0 || valid <= 0 || ncols < valid || ncols > lds || ncols > ldp)
        return fail(IG_EINVAL, "bad softmax sizes rows=%d valid=%d ncols=%d lds=%d ldp=%d", rows,
                    valid, ncols, lds, ldp);
    if (lds % 4 || ldp % 4) return fail(IG_EUNSUPPORTED, "lds and ldp must be multiples of 4");
    if (rows == 0) return IG_OK;
    int r;
    if ((r = check_ptr(S, "S")) || (r = check_ptr(P, "P", false))) return r;
    if ((uintptr_t)P & 7) return fail(IG_EINVAL, "P is not 8-byte aligned");
    (void)hipGetLastError();
    launch_softmax(S, rows, lds, valid, ncols, reinterpret_cast<_Float16 *>(P), ldp,
                   reinterpret_cast<hipStream_t>(stream));
    return check_launch("softmax launch");
}

size_t ig_attention_workspace_bytes(int m, int C)
{
    clear_error();
    const bool width_ok = C == 128 || C == 256 || C == 384 || C == 512;
    if (m <= 0 || !width_ok) {
        fail(!width_ok ? IG_EUNSUPPORTED : IG_EINVAL, "attention m=%d C=%d (C must be 128, 256, 384 or 512)", m, C);
        return 0;
    }
    return flash_workspace_bytes(m, C);
}

int attention_f16(const uint16_t *q, const uint16_t *k, const uint16_t *vt, int m, int ld, int C,
                  const float *bv, void *ws, size_t ws_bytes, uint16_t *out, void *stream)
{
    clear_error();
    if (m <= 0 || m >= (1 << 22)) return fail(IG_EINVAL, "attention m=%d outside 1..2^22-1", m);
    if (C != 128 && C != 256 && C != 384 && C != 512)
        return fail(IG_EUNSUPPORTED, "attention width %d: the single-pass kernel takes 128, 256, 384 or 512", C);
    if (!flash_supported(m, ld, C))
        return fail(IG_EINVAL, "ld=%d must be >= m rounded up to 32 (%d), a multiple of 8, and ld*C*2 below %lld bytes",
                    ld, (m + 31) / 32 * 32, (long long)kConvInMaxBytes);
    int r;
    if ((r = check_ptr(q, "q", true)) || (r = check_ptr(k, "k", true)) || (r = check_ptr(vt, "vt", true)) ||
        (r = check_ptr(out, "out", true)))
        return r;
    if (bv && (r = check_ptr(bv, "bv", true))) return r;
    const size_t need = flash_workspace_bytes(m, C);
    if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 15)))
        return fail(IG_EWORKSPACE, "attention workspace of %zu bytes, %zu needed (16-byte aligned)", ws_bytes, need);
    FlashArgs a{};
    a.q = reinterpret_cast<const _Float16 *>(q);
    a.k = reinterpret_cast<const _Float16 *>(k);
    a.vt = reinterpret_cast<const _Float16 *>(vt);
    a.ld = ld;
    a.m = m;
    a.c = C;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)C));
    a.bv = bv;
    a.out = reinterpret_cast<_Float16 *>(out);
    (void)hipGetLastError();
    launch_flash(a, ws, reinterpret_cast<hipStream_t>(stream));
    return check_launch("attention launch");
}

int ig_latent_to_nhwc_f16(const float *z, int zc, int M, int cp, uint16_t *y, void *stream)
{
    clear_error();
    if (M < 0 || zc <= 0 || cp < zc || cp % 8) return fail(IG_EINVAL, "bad latent sizes zc=%d cp=%d", zc, cp);
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(z, "z", false)) || (r = check_ptr(y, "y"))) return r;
    (void)hipGetLastError();
    launch_latent_ingest(z, zc, M, cp, reinterpret_cast<_Float16 *>(y),
                         reinterpret_cast<hipStream_t>(stream));
    return check_launch("latent launch");
}

int ig_nhwc_to_nchw(const float *y, int M, int ld, int nch, const float *bias, float *out,
                    void *stream)
{
    clear_error();
    if (M < 0 || nch <= 0 || ld < nch) return fail(IG_EINVAL, "bad output sizes nch=%d ld=%d", nch, ld);
    if (M == 0) return IG_OK;
    int r;
    if ((r = check_ptr(y, "y", false)) || (r = check_ptr(out, "out", false))) return r;
    (void)hipGetLastError();
    launch_nhwc_to_nchw(y, M, ld, nch, bias, out, reinterpret_cast<hipStream_t>(stream));
    return check_launch("output launch");
}

int ig_conv3x3_out_nchw(const uint16_t *x, int H, int W, int cin_p, const uint16_t *w, int cout, int cout_p,
                        const float *bias, float *out, void *stream)
{
    clear_error();
    if (H < 0 || W < 0) return fail(IG_EINVAL, "bad image %dx%d", H, W);
    if (cin_p <= 0 || cin_p % 64 || cout <= 0 || cout_p < cout || cout_p % 64)
        return fail(IG_EINVAL, "bad channel counts cin_p=%d cout=%d cout_p=%d", cin_p, cout, cout_p);
    if (cout > 16) return fail(IG_EUNSUPPORTED, "output conv takes at most 16 channels, got %d", cout);
    if ((int64_t)H * W * cin_p * 2 >= (3LL << 30)) return fail(IG_EUNSUPPORTED, "input too large");
    if ((int64_t)H * W == 0) return IG_OK;
    int r;
    if ((r = check_ptr(x, "x", true)) || (r = check_ptr(w, "w", true)) || (r = check_ptr(out, "out", false)))
        return r;
    (void)hipGetLastError();
    launch_conv_out(reinterpret_cast<const _Float16 *>(x), H, W, cin_p, reinterpret_cast<const _Float16 *>(w),
                    cout, cout_p, bias, out, reinterpret_cast<hipStream_t>(stream));
    return check_launch("output conv launch");
}

int ig_zero_rows_f16(uint16_t *y, int r0, int r1, int ld, void *stream)
{
    clear_error();
    if (r0 < 0 || r1 < r0 || ld <= 0) return fail(IG_EINVAL, "bad row range");
    if (r1 == r0) return IG_OK;
    if (!y) return fail(IG_EINVAL, "y is NULL");
    (void)hipGetLastError();
    launch_zero_rows_f16(reinterpret_cast<_Float16 *>(y), r0, r1, ld,
                         reinterpret_cast<hipStream_t>(stream));
    return check_launch("fill launch");
}

int ig_dupup_add(const float *src, int H, int W, int cin_p, float *x, int cout, int cout_p,
                 int factor, int repeats, int ft, void *stream)
{
    clear_error();
    if (H < 0 || W < 0 || cin_p <= 0 || cout <= 0 || cout_p < cout || factor <= 0 || repeats <= 0 || ft < 1)
        return fail(IG_EINVAL, "bad DupUp arguments");
    const int64_t jmax = ((int64_t)(cout - 1) * factor + (int64_t)(ft - 1) * 4 + 3) / repeats;
    if (jmax >= cin_p) return fail(IG_EINVAL, "shuffled channel %lld outside cin_p=%d", (long long)jmax, cin_p);
    if (cout_p % 4) return fail(IG_EUNSUPPORTED, "cout_p=%d must be a multiple of 4", cout_p);
    if ((int64_t)4 * H * W * cout_p >= (1LL << 40)) return fail(IG_EUNSUPPORTED, "too many elements");
    if (H == 0 || W == 0) return IG_OK;
    int r;
    if ((r = check_ptr(src, "src", false)) || (r = check_ptr(x, "x"))) return r;
    (void)hipGetLastError();
    launch_dupup(src, H, W, cin_p, x, cout, cout_p, factor, repeats, ft, reinterpret_cast<hipStream_t>(stream));
    return check_launch("dupup launch");
}

}  // extern "C"
