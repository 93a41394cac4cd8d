// decoder_forward: the whole image-VAE decoder on one stream, every tensor
// resident in HBM (page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs":
// `decode`, `Rec::resnet`, `attention`, `run_blocks`, `output_rows`; page
// "cortiq-engine 0.7.6, src/vae.rs": `VaeDecoder::decode` for the order
// conv_in -> mid resnet -> attention -> mid resnet -> up stages -> norm_out
// -> conv_out).
//
// Differences from the pages' recording, chosen for one MI355X:
//  * the whole frame runs at once (no horizontal bands: the largest tensor
//    of a 2048^2 decode is 2.1 GB, far inside 288 GB of HBM);
//  * the combine passes are folded into conv epilogues: the up conv and
//    conv_in write x = oscale*acc + b directly, the second conv of a
//    resnet adds into the stream (x += acc + b2), and a shortcut writes
//    x = 2^g*acc + b_sc before that add -- two f32 stream passes fewer per
//    resnet unit;
//  * q and k leave their GEMMs as f16 with the bias added (the pages' conv
//    then cast(+bias)), and the attention output projection adds into x;
//  * the chunk's f32 score matrix is never stored: a first GEMM pass keeps
//    only per-row softmax statistics, a second recomputes the same scores
//    and writes P directly (the same P, without 6 bytes per score of HBM
//    traffic).
#include <cmath>

#include "ig_internal.h"

namespace ig {
namespace {

constexpr size_t kAlign = 256;
inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
constexpr float kEps = 1e-12f;

struct Plan {
    int64_t max_x = 0;   // f32 stream elements
    int64_t max_h = 0;   // f32 conv outputs
    int64_t max_xn = 0;  // f16 conv inputs
    int64_t max_xg = 0;  // f16 guarded shortcut input
    int m = 0, mp = 0, C = 0, qc = 0;
    bool flash = false;  // single-pass attention (else query chunks)
    int H = 0, W = 0;    // output frame
    size_t off_x, off_h, off_xn, off_xg, off_q, off_k, off_vt, off_o, off_s, off_p, total;
};

int check_conv_w(const ig_conv_w &c, const char *name, int k)
{
    if (!c.w || !aligned16(c.w)) return fail(IG_EINVAL, "%s: weight plane NULL or not 16-byte aligned", name);
    if (c.b && !aligned16(c.b)) return fail(IG_EINVAL, "%s: bias not 16-byte aligned", name);
    if (c.k != k) return fail(IG_EUNSUPPORTED, "%s: k=%d, expected %d", name, c.k, k);
    if (c.cin <= 0 || c.cout <= 0 || c.cin > c.cin_p || c.cout > c.cout_p)
        return fail(IG_EINVAL, "%s: bad channel counts %d/%d -> %d/%d", name, c.cin, c.cin_p, c.cout, c.cout_p);
    if (c.cin_p % 64 || c.cout_p % 64) return fail(IG_EUNSUPPORTED, "%s: padded widths must be multiples of 64", name);
    return IG_OK;
}

int check_gamma(const float *g, const char *name)
{
    if (!g || !aligned16(g)) return fail(IG_EINVAL, "%s: gamma NULL or not 16-byte aligned", name);
    return IG_OK;
}

inline void upd(int64_t &m, int64_t v)
{
    if (v > m) m = v;
}

// Check one resnet against the incoming width (c, cp) and update the plan
// for M pixels; returns the outgoing width through c, cp.
int plan_resnet(const ig_resnet_w &r, const char *name, int &c, int &cp, int64_t M, Plan &pl)
{
    int e;
    if ((e = check_gamma(r.g1, name)) || (e = check_gamma(r.g2, name))) return e;
    if ((e = check_conv_w(r.c1, name, 3)) || (e = check_conv_w(r.c2, name, 3))) return e;
    if (r.c1.cin != c || r.c1.cin_p != cp) return fail(IG_EINVAL, "%s: conv1 input %d/%d, stream is %d/%d", name, r.c1.cin, r.c1.cin_p, c, cp);
    if (r.c2.cin != r.c1.cout || r.c2.cin_p != r.c1.cout_p || r.c2.cout != r.c1.cout || r.c2.cout_p != r.c1.cout_p)
        return fail(IG_EINVAL, "%s: conv2 must map conv1's width to itself", name);
    if (r.has_sc) {
        if ((e = check_conv_w(r.sc, name, 1))) return e;
        if (r.sc.cin != c || r.sc.cin_p != cp || r.sc.cout != r.c2.cout || r.sc.cout_p != r.c2.cout_p)
            return fail(IG_EINVAL, "%s: shortcut must map %d -> %d", name, c, r.c2.cout);
        upd(pl.max_xg, M * cp);
    } else if (r.c2.cout != c || r.c2.cout_p != cp) {
        return fail(IG_EINVAL, "%s: width changes %d -> %d without a shortcut", name, c, r.c2.cout);
    }
    upd(pl.max_xn, M * cp);
    upd(pl.max_xn, M * r.c1.cout_p);
    upd(pl.max_h, M * r.c1.cout_p);
    upd(pl.max_x, M * cp);
    upd(pl.max_x, M * r.c2.cout_p);
    c = r.c2.cout;
    cp = r.c2.cout_p;
    return IG_OK;
}

int make_plan(const ig_decoder *d, int h0, int w0, int q_chunk, Plan &pl)
{
    if (!d) return fail(IG_EINVAL, "decoder descriptor is NULL");
    if (h0 <= 0 || w0 <= 0) return fail(IG_EINVAL, "latent size %dx%d", h0, w0);
    if (d->zc <= 0) return fail(IG_EINVAL, "zc=%d", d->zc);
    if (d->n_up < 0 || d->n_up > IG_MAX_UP) return fail(IG_EINVAL, "n_up=%d outside 0..%d", d->n_up, IG_MAX_UP);
    int e;
    if ((e = check_conv_w(d->conv_in, "conv_in", 3))) return e;
    if (d->conv_in.cin != d->zc) return fail(IG_EINVAL, "conv_in takes %d channels, latent has %d", d->conv_in.cin, d->zc);
    int H = h0, W = w0;
    int64_t M = (int64_t)H * W;
    upd(pl.max_xn, M * d->conv_in.cin_p);
    int c = d->conv_in.cout, cp = d->conv_in.cout_p;
    upd(pl.max_x, M * cp);
    if ((e = plan_resnet(d->mid[0], "mid.0", c, cp, M, pl))) return e;
    // attention over the M latent pixels at width c (unpadded)
    const ig_attn_w &a = d->attn;
    if ((e = check_gamma(a.gamma, "attn"))) return e;
    const ig_conv_w *aw[4] = {&a.q, &a.k, &a.v, &a.proj};
    const char *an[4] = {"attn.q", "attn.k", "attn.v", "attn.proj"};
    if (cp != c || c % 64) return fail(IG_EUNSUPPORTED, "attention width %d must be unpadded and a multiple of 64", c);
    for (int i = 0; i < 4; ++i) {
        if ((e = check_conv_w(*aw[i], an[i], 1))) return e;
        if (aw[i]->cin != c || aw[i]->cout != c || aw[i]->cin_p != c || aw[i]->cout_p != c)
            return fail(IG_EINVAL, "%s must map %d -> %d unpadded", an[i], c, c);
    }
    if (M >= (1LL << 30)) return fail(IG_EUNSUPPORTED, "latent too large for the attention");
    pl.m = (int)M;
    pl.mp = (int)((M + 63) / 64 * 64);
    pl.C = c;
    pl.flash = q_chunk <= 0 && flash_supported(pl.m, pl.mp, c);
    pl.qc = q_chunk > 0 ? q_chunk : 16384;
    if (pl.qc > pl.m) pl.qc = pl.m;
    upd(pl.max_xn, (int64_t)pl.mp * c);
    if (!pl.flash && (uint64_t)pl.qc * pl.mp * 2 >= (3ULL << 30))
        return fail(IG_EUNSUPPORTED, "query chunk %d x %d keys: probabilities exceed 3 GiB; pass a smaller q_chunk", pl.qc, pl.mp);
    if ((e = plan_resnet(d->mid[1], "mid.1", c, cp, M, pl))) return e;
    for (int s = 0; s < d->n_up; ++s) {
        const ig_up_w &u = d->ups[s];
        if (u.n_res < 0 || u.n_res > IG_MAX_RES) return fail(IG_EINVAL, "ups[%d].n_res=%d", s, u.n_res);
        for (int r = 0; r < u.n_res; ++r) {
            char nm[32];
            snprintf(nm, sizeof nm, "ups.%d.res.%d", s, r);
            if ((e = plan_resnet(u.res[r], nm, c, cp, M, pl))) return e;
        }
        if (u.has_up) {
            char nm[32];
            snprintf(nm, sizeof nm, "ups.%d.up", s);
            if ((e = check_conv_w(u.up, nm, 3))) return e;
            if (u.up.cin != c || u.up.cin_p != cp) return fail(IG_EINVAL, "%s: input %d, stream %d", nm, u.up.cin, c);
            upd(pl.max_xn, M * cp);
            upd(pl.max_xg, M * cp);
            H *= 2;
            W *= 2;
            M *= 4;
            if (M >= (1LL << 31)) return fail(IG_EUNSUPPORTED, "frame too large");
            c = u.up.cout;
            cp = u.up.cout_p;
            upd(pl.max_x, M * cp);
        }
    }
    if ((e = check_gamma(d->norm_out_gamma, "norm_out"))) return e;
    if (d->norm_out_c != c) return fail(IG_EINVAL, "norm_out has %d channels, stream %d", d->norm_out_c, c);
    if ((e = check_conv_w(d->conv_out, "conv_out", 3))) return e;
    if (d->conv_out.cin != c || d->conv_out.cin_p != cp) return fail(IG_EINVAL, "conv_out input %d, stream %d", d->conv_out.cin, c);
    upd(pl.max_xn, M * cp);
    if (d->conv_out.cout > 16) upd(pl.max_h, M * d->conv_out.cout_p);  // else straight to the frame
    pl.H = H;
    pl.W = W;
    // layout
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += round_up(bytes);
        return at;
    };
    const int64_t mp = pl.mp, C = pl.C, qc = pl.qc;
    pl.off_x = take(pl.max_x * 4);
    pl.off_h = take(pl.max_h * 4);
    pl.off_xn = take(pl.max_xn * 2);
    pl.off_xg = take(pl.max_xg * 2);
    pl.off_q = take(mp * C * 2);
    pl.off_k = take(mp * C * 2);
    pl.off_vt = take(C * mp * 2);
    if (pl.flash) {
        // the single-pass kernel's key-range partials (if any)
        pl.off_o = take(0);
        pl.off_s = take(flash_workspace_bytes(pl.m));
        pl.off_p = take(0);
    } else {
        pl.off_o = take(mp * C * 4);
        // per-row partial softmax statistics of a query chunk, then the
        // rows' final (max, 1 / sum)
        pl.off_s = take((qc * gemm2_stat_parts((int)mp) * 2 + qc * 2) * 4);
        pl.off_p = take(qc * mp * 2);
    }
    pl.total = o;
    return IG_OK;
}

struct Run {
    hipStream_t s;
    char *ws;
    const Plan &pl;
    int g;
    float *x, *h, *o32, *S;
    _Float16 *xn, *xg, *q16, *k16, *vt16, *P;

    void conv(int mode, const _Float16 *in, int H, int W, const ig_conv_w &cw, const float *bias,
              float oscale, int acc, float *out)
    {
        IgemmArgs a{};
        a.a = in;
        a.b = reinterpret_cast<const _Float16 *>(cw.w);
        a.bias = bias;
        a.c = out;
        a.M = H * W * (mode == kConv3x3Up2 ? 4 : 1);
        a.N = cw.cout_p;
        a.K = (mode == kGemm ? 1 : 9) * cw.cin_p;
        a.lda = cw.cin_p;
        a.ldb = a.K;
        a.ldc = cw.cout_p;
        a.H = H;
        a.W = W;
        a.cin_p = cw.cin_p;
        a.oscale = oscale;
        a.accumulate = acc;
        a.out_f16 = 0;
        launch_igemm(mode, a, s);
    }

    // a 3x3 conv whose epilogue emits f16(RMS_norm(oscale*acc + bias; gamma) -> SiLU)
    // instead of the f32 result (every channel of a pixel in one tile)
    void conv_norm(int mode, const _Float16 *in, int H, int W, const ig_conv_w &cw, const float *bias,
                   float oscale, const float *gamma, int c_real, _Float16 *yn)
    {
        IgemmArgs a{};
        a.a = in;
        a.b = reinterpret_cast<const _Float16 *>(cw.w);
        a.bias = bias;
        a.c = nullptr;
        a.M = H * W * (mode == kConv3x3Up2 ? 4 : 1);
        a.N = cw.cout_p;
        a.K = 9 * cw.cin_p;
        a.lda = cw.cin_p;
        a.ldb = a.K;
        a.ldc = cw.cout_p;
        a.H = H;
        a.W = W;
        a.cin_p = cw.cin_p;
        a.oscale = oscale;
        a.ngamma = gamma;
        a.ny = yn;
        a.norm_c = c_real;
        a.norm_silu = 1;
        a.norm_eps = kEps;
        a.write_out = 0;
        launch_conv_halo(mode, a, s);
    }
    static bool fusable(const ig_conv_w &cw) { return cw.cout_p == 64 || cw.cout_p == 128; }

    void gemm(const _Float16 *A, int M, int K, int lda, const _Float16 *B, int N, int ldb,
              const float *bias, float oscale, void *C, int ldc, int f16, int acc)
    {
        IgemmArgs a{};
        a.a = A;
        a.b = B;
        a.bias = bias;
        a.c = C;
        a.M = M;
        a.N = N;
        a.K = K;
        a.lda = lda;
        a.ldb = ldb;
        a.ldc = ldc;
        a.oscale = oscale;
        a.accumulate = acc;
        a.out_f16 = f16;
        launch_igemm(kGemm, a, s);
    }

    // Rec::resnet with the combines folded into the epilogues
    void resnet(const ig_resnet_w &r, int H, int W, int cp)
    {
        const int M = H * W;
        launch_rmsnorm(x, M, cp, r.c1.cin, nullptr, r.g1, 1, kEps, xn, s);
        if (r.has_sc) {
            launch_guard_cast(x, M, cp, nullptr, g, xg, s);
            conv(kGemm, xg, H, W, r.sc, r.sc.b, ldexpf(1.f, g), 0, x);
        }
        if (fusable(r.c1)) {
            // conv1's epilogue normalises (h + b1) itself; the f16 result
            // goes to the h region (conv1 still reads xn)
            _Float16 *hn = reinterpret_cast<_Float16 *>(h);
            conv_norm(kConv3x3, xn, H, W, r.c1, r.c1.b, 1.f, r.g2, r.c1.cout, hn);
            conv(kConv3x3, hn, H, W, r.c2, r.c2.b, 1.f, 1, x);
        } else {
            conv(kConv3x3, xn, H, W, r.c1, nullptr, 1.f, 0, h);
            launch_rmsnorm(h, M, r.c1.cout_p, r.c1.cout, r.c1.b, r.g2, 1, kEps, xn, s);
            conv(kConv3x3, xn, H, W, r.c2, r.c2.b, 1.f, 1, x);
        }
    }

    // the mid attention, single head over the m latent pixels
    void attention(const ig_attn_w &a)
    {
        const int m = pl.m, mp = pl.mp, C = pl.C, qc = pl.qc;
        launch_rmsnorm(x, m, C, C, nullptr, a.gamma, 0, kEps, xn, s);
        launch_zero_rows_f16(xn, m, mp, C, s);
        const _Float16 *wq = reinterpret_cast<const _Float16 *>(a.q.w);
        const _Float16 *wk = reinterpret_cast<const _Float16 *>(a.k.w);
        const _Float16 *wv = reinterpret_cast<const _Float16 *>(a.v.w);
        const _Float16 *wp = reinterpret_cast<const _Float16 *>(a.proj.w);
        gemm(xn, mp, C, C, wq, C, C, a.q.b, 1.f, q16, C, 1, 0);
        gemm(xn, mp, C, C, wk, C, C, a.k.b, 1.f, k16, C, 1, 0);
        // V^T [C][mp] = Wv . xn^T; V's bias comes after P.V (P's rows sum to 1)
        gemm(wv, C, C, C, xn, mp, C, nullptr, 1.f, vt16, mp, 1, 0);
        if (pl.flash) {
            // one pass over the keys, f16(O + bv) straight into xn
            FlashArgs f{};
            f.q = q16;
            f.k = k16;
            f.vt = vt16;
            f.ld = mp;
            f.m = m;
            f.scale_log2 = (float)(1.4426950408889634 / sqrt((double)C));
            f.bv = a.v.b;
            f.out = xn;
            launch_flash(f, S, s);
            gemm(xn, m, C, C, wp, C, C, a.proj.b, 1.f, x, C, 0, 1);
            return;
        }
        const float scale = 1.0f / sqrtf((float)C);
        // per chunk: the scores' row statistics, then P, never storing the
        // scores themselves; then O = P.V
        const int nparts = gemm2_stat_parts(mp);
        float *rowstat = S + (int64_t)qc * nparts * 2;
        for (int q0 = 0; q0 < m; q0 += qc) {
            const int rows = (m - q0) < qc ? (m - q0) : qc;
            Gemm2Args g{};
            g.a = q16 + (int64_t)q0 * C;
            g.b = k16;
            g.M = rows;
            g.N = mp;
            g.K = C;
            g.lda = C;
            g.ldb = C;
            g.valid = m;
            g.oscale = scale;
            g.stats = S;
            launch_gemm2(kEpiStats, g, s);
            launch_rowstat(S, nparts, rows, rowstat, s);
            g.c = P;
            g.ldc = mp;
            g.rowstat = rowstat;
            launch_gemm2(kEpiProb, g, s);
            gemm(P, rows, mp, mp, vt16, C, mp, nullptr, 1.f, o32 + (int64_t)q0 * C, C, 0, 0);
        }
        launch_guard_cast(o32, m, C, a.v.b, 0, xn, s);
        gemm(xn, m, C, C, wp, C, C, a.proj.b, 1.f, x, C, 0, 1);
    }
};

}  // namespace
}  // namespace ig

using namespace ig;

extern "C" {

size_t ig_decoder_workspace_bytes(const ig_decoder *dec, int h0, int w0, int q_chunk)
{
    clear_error();
    Plan pl;
    if (make_plan(dec, h0, w0, q_chunk, pl)) return 0;
    return pl.total;
}

int decoder_forward(const ig_decoder *dec, const float *latent, int h0, int w0, int guard_log2,
                    int q_chunk, void *ws, size_t ws_bytes, float *out, void *stream)
{
    clear_error();
    Plan pl;
    int e = make_plan(dec, h0, w0, q_chunk, pl);
    if (e) return e;
    if (guard_log2 < 0 || guard_log2 > 14) return fail(IG_EINVAL, "guard_log2=%d outside 0..14", guard_log2);
    if (!latent || !out) return fail(IG_EINVAL, "latent or out is NULL");
    if (!ws || ((uintptr_t)ws & (kAlign - 1))) return fail(IG_EWORKSPACE, "workspace NULL or not 256-byte aligned");
    if (ws_bytes < pl.total) return fail(IG_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, pl.total);
    const ig_decoder &d = *dec;
    char *w = reinterpret_cast<char *>(ws);
    Run r{reinterpret_cast<hipStream_t>(stream), w, pl, guard_log2,
          reinterpret_cast<float *>(w + pl.off_x), reinterpret_cast<float *>(w + pl.off_h),
          reinterpret_cast<float *>(w + pl.off_o), reinterpret_cast<float *>(w + pl.off_s),
          reinterpret_cast<_Float16 *>(w + pl.off_xn), reinterpret_cast<_Float16 *>(w + pl.off_xg),
          reinterpret_cast<_Float16 *>(w + pl.off_q), reinterpret_cast<_Float16 *>(w + pl.off_k),
          reinterpret_cast<_Float16 *>(w + pl.off_vt), reinterpret_cast<_Float16 *>(w + pl.off_p)};
    hipStream_t s = r.s;
    (void)hipGetLastError();
    int H = h0, W = w0;
    // latent -> f16 NHWC -> conv_in, x = conv + b
    launch_latent_ingest(latent, d.zc, H * W, d.conv_in.cin_p, r.xn, s);
    r.conv(kConv3x3, r.xn, H, W, d.conv_in, d.conv_in.b, 1.f, 0, r.x);
    int cp = d.conv_in.cout_p;
    r.resnet(d.mid[0], H, W, cp);
    cp = d.mid[0].c2.cout_p;
    r.attention(d.attn);
    r.resnet(d.mid[1], H, W, cp);
    cp = d.mid[1].c2.cout_p;
    const float gs = ldexpf(1.f, guard_log2);
    bool normed = false;
    for (int st = 0; st < d.n_up; ++st) {
        const ig_up_w &u = d.ups[st];
        for (int k = 0; k < u.n_res; ++k) {
            r.resnet(u.res[k], H, W, cp);
            cp = u.res[k].c2.cout_p;
        }
        if (u.has_up) {
            launch_guard_cast(r.x, H * W, cp, nullptr, guard_log2, r.xg, s);
            if (st == d.n_up - 1 && Run::fusable(u.up) && d.norm_out_c == u.up.cout) {
                // the last up conv's epilogue applies norm_out + SiLU; the
                // f32 stream is not needed after it
                r.conv_norm(kConv3x3Up2, r.xg, H, W, u.up, u.up.b, gs, d.norm_out_gamma, d.norm_out_c, r.xn);
                normed = true;
            } else {
                r.conv(kConv3x3Up2, r.xg, H, W, u.up, u.up.b, gs, 0, r.x);
            }
            H *= 2;
            W *= 2;
            cp = u.up.cout_p;
        }
    }
    if (!normed) launch_rmsnorm(r.x, H * W, cp, d.norm_out_c, nullptr, d.norm_out_gamma, 1, kEps, r.xn, s);
    if (d.conv_out.cout <= 16) {
        // few output channels: straight into the NCHW frame
        launch_conv_out(r.xn, H, W, d.conv_out.cin_p, reinterpret_cast<const _Float16 *>(d.conv_out.w),
                        d.conv_out.cout, d.conv_out.cout_p, d.conv_out.b, out, s);
    } else {
        r.conv(kConv3x3, r.xn, H, W, d.conv_out, d.conv_out.b, 1.f, 0, r.h);
        launch_nhwc_to_nchw(r.h, H * W, d.conv_out.cout_p, d.conv_out.cout, nullptr, out, s);
    }
    return check_launch("decoder_forward");
}

}  // extern "C"
