// decoder_forward: the whole image-VAE decoder on one stream, every tensor
// resident in HBM (page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs":
// `decode`, `Rec::resnet`, `attention`, `run_blocks`, `output_rows`; page
// "cortiq-engine 0.7.6, src/vae.rs": `VaeDecoder::decode` for the order
// conv_in -> mid resnet -> attention -> mid resnet -> up stages -> norm_out
// -> conv_out).
//
// Differences from the pages' recording, chosen for one MI355X:
//  * decoder_forward runs the whole frame at once (the largest tensor of a
//    2048^2 decode is 2.1 GB, far inside 288 GB of HBM); decoder_forward_bands
//    runs the up blocks from a chosen one on in horizontal bands with exact
//    halos, as the pages do to bound memory (page "cortiq-engine 0.8.3,
//    src/gpu_wgpu/qi21_vae.rs", the bands section, `run_blocks`,
//    `output_rows`); each kept pixel goes through the same kernels with the
//    same inputs as in the whole frame, so the two outputs are identical;
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

// A contiguous range of image rows [first, end) at one resolution of the
// up path.
struct Span {
    int first = 0, end = 0;
    int rows() const { return end - first; }
};

// One operation of the up path, seen from the rows it produces: a 3x3 conv
// on a level of `height` rows, or the nearest-2x upsample that a block
// `block` ends with (its output level has twice the rows of its input).
struct PathStep {
    bool upsample;
    int height;
    int block;
};

// The rows one step reads to produce the rows `out`: a 3x3 conv one more on
// each side, cut at the level's edges (there the zero padding is the frame's
// own); an upsample the source rows of out's rows, row r coming from r / 2.
Span read_rows(const PathStep &p, Span out)
{
    if (p.upsample) return Span{out.first / 2, (out.end + 1) / 2};
    return Span{out.first > 0 ? out.first - 1 : 0, out.end < p.height ? out.end + 1 : p.height};
}

// Band planning by receptive fields: list the steps from block s's input to
// the frame (each block: 2 n_res 3x3 convs, then, with has_up, the upsample
// and its 3x3 conv; conv_out last), then fold the kept output rows back
// through them. input: the rows of block s's input the band needs; feed[i]:
// the rows block i (i >= s, with has_up) hands to its upsample.
void plan_band(int n_up, const int *n_res, const int *has_up, int h0, int s, Span keep, Span &input, Span *feed)
{
    PathStep steps[IG_MAX_UP * (2 * IG_MAX_RES + 2) + 1];
    int n = 0, height = h0;
    for (int i = 0; i < s; ++i)
        if (has_up[i]) height *= 2;
    for (int i = s; i < n_up; ++i) {
        for (int k = 0; k < 2 * n_res[i]; ++k) steps[n++] = PathStep{false, height, i};
        if (has_up[i]) {
            steps[n++] = PathStep{true, 0, i};
            height *= 2;
            steps[n++] = PathStep{false, height, i};
        }
    }
    steps[n++] = PathStep{false, height, -1};  // conv_out
    for (int i = 0; i < n_up; ++i) feed[i] = Span{};
    Span span = keep;
    for (int j = n - 1; j >= 0; --j) {
        span = read_rows(steps[j], span);
        if (steps[j].upsample) feed[steps[j].block] = span;
    }
    input = span;
}

struct Plan {
    int64_t max_x = 0;   // f32 stream elements (the whole frame's)
    int64_t max_xb = 0;  // f32 stream elements of a band
    int64_t max_h = 0;   // f32 conv outputs
    int64_t max_xn = 0;  // f16 conv inputs
    int64_t max_xg = 0;  // f16 guarded shortcut input
    int64_t max_cp = 0;  // f32 up-stage input kept for its DupUp shortcut
    int gn_groups = 0;   // GroupNorm's groups (0: RMS_norm)
    float gn_eps = 0.f;
    size_t max_gn = 0;   // bytes of GroupNorm's per-chunk statistics
    size_t gn_part = 0;  // bytes of one set of conv-gathered GroupNorm partials
    int m = 0, mp = 0, C = 0, qc = 0;
    bool flash = false;  // single-pass attention (else query chunks)
    int H = 0, W = 0;    // output frame
    int s = 0;           // up blocks s.. run in bands (s == n_up: none)
    int band_rows = 0;   // kept output rows per band
    size_t off_x, off_xb, off_h, off_xn, off_xg, off_q, off_k, off_vt, off_o, off_s, off_p, off_cp, off_gn, total;
    size_t off_gpx = 0, off_gph = 0, off_gtab = 0;  // GroupNorm partials of x and h, the per-channel table
};

int check_conv_w(const ig_conv_w &c, const char *name, int k)
{
    if (!c.w || !aligned16(c.w)) return fail(IG_EINVAL, "%s: weight plane NULL or not 16-byte aligned", name);
    if (c.b && !aligned16(c.b)) return fail(IG_EINVAL, "%s: bias not 16-byte aligned", name);
    if (c.k != k) return fail(IG_EUNSUPPORTED, "%s: k=%d, expected %d", name, c.k, k);
    if (c.cin <= 0 || c.cout <= 0 || c.cin > c.cin_p || c.cout > c.cout_p)
        return fail(IG_EINVAL, "%s: bad channel counts %d/%d -> %d/%d", name, c.cin, c.cin_p, c.cout, c.cout_p);
    if (c.cin_p % 64 || c.cout_p % 64) return fail(IG_EUNSUPPORTED, "%s: padded widths must be multiples of 64", name);
    if (c.cin_p > kConvMaxChannels || c.cout_p > kConvMaxChannels)
        return fail(IG_EUNSUPPORTED, "%s: padded widths above %d", name, kConvMaxChannels);
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

// Check one resnet against the incoming width (c, cp); returns the outgoing
// width through c, cp.
// the decoder's norm kind and GroupNorm's groups (0 with RMS_norm)
struct NormCfg {
    int groups = 0;
};

// a GroupNorm site: its beta, and its widths within the kernel's reach
int check_gn_site(const NormCfg &nc, const float *beta, int c, int cp, const char *name)
{
    if (!nc.groups) return IG_OK;
    if (!beta || !aligned16(beta)) return fail(IG_EINVAL, "%s: GroupNorm beta NULL or not 16-byte aligned", name);
    if (!gn_supported(cp, c, nc.groups))
        return fail(IG_EUNSUPPORTED, "%s: GroupNorm(%d) over %d channels padded to %d", name, nc.groups, c, cp);
    return IG_OK;
}

int check_resnet(const ig_resnet_w &r, const char *name, int &c, int &cp, const NormCfg &nc)
{
    int e;
    if ((e = check_gamma(r.g1, name)) || (e = check_gamma(r.g2, name))) return e;
    if ((e = check_gn_site(nc, r.beta1, c, cp, name))) return e;
    if ((e = check_gn_site(nc, r.beta2, r.c1.cout, r.c1.cout_p, name))) return e;
    if ((e = check_conv_w(r.c1, name, 3)) || (e = check_conv_w(r.c2, name, 3))) return e;
    if (r.c1.cin != c || r.c1.cin_p != cp) return fail(IG_EINVAL, "%s: conv1 input %d/%d, stream is %d/%d", name, r.c1.cin, r.c1.cin_p, c, cp);
    if (r.c2.cin != r.c1.cout || r.c2.cin_p != r.c1.cout_p || r.c2.cout != r.c1.cout || r.c2.cout_p != r.c1.cout_p)
        return fail(IG_EINVAL, "%s: conv2 must map conv1's width to itself", name);
    if (r.has_sc) {
        if ((e = check_conv_w(r.sc, name, 1))) return e;
        if (r.sc.cin != c || r.sc.cin_p != cp || r.sc.cout != r.c2.cout || r.sc.cout_p != r.c2.cout_p)
            return fail(IG_EINVAL, "%s: shortcut must map %d -> %d", name, c, r.c2.cout);
    } else if (r.c2.cout != c || r.c2.cout_p != cp) {
        return fail(IG_EINVAL, "%s: width changes %d -> %d without a shortcut", name, c, r.c2.cout);
    }
    c = r.c2.cout;
    cp = r.c2.cout_p;
    return IG_OK;
}

// the buffers one resnet on M pixels uses; xmax: the stream's maximum
// GroupNorm's statistics for a site of M pixels, cp channels
void size_gn(int64_t M, int cp, Plan &pl)
{
    if (pl.gn_groups && M > 0) {
        const size_t b = gn_workspace_bytes((int)M, cp, pl.gn_groups);
        if (b > pl.max_gn) pl.max_gn = b;
    }
}

void size_resnet(const ig_resnet_w &r, int64_t M, int cp, int64_t &xmax, Plan &pl)
{
    size_gn(M, cp, pl);
    size_gn(M, r.c1.cout_p, pl);
    if (r.has_sc) upd(pl.max_xg, M * cp);
    upd(pl.max_xn, M * cp);
    upd(pl.max_xn, M * r.c1.cout_p);
    upd(pl.max_h, M * r.c1.cout_p);
    upd(xmax, M * cp);
    upd(xmax, M * r.c2.cout_p);
}

// the up blocks' real and padded widths at their inputs and outputs
struct Widths {
    int cp_in[IG_MAX_UP], cp_out[IG_MAX_UP];
};

// Check the whole descriptor; frame sizes to pl.H, pl.W.
int check_decoder(const ig_decoder *d, int h0, int w0, Widths &wd, Plan &pl)
{
    if (!d) return fail(IG_EINVAL, "decoder descriptor is NULL");
    if (h0 <= 0 || w0 <= 0) return fail(IG_EINVAL, "latent size %dx%d", h0, w0);
    if (d->zc <= 0) return fail(IG_EINVAL, "zc=%d", d->zc);
    if (d->n_up < 0 || d->n_up > IG_MAX_UP) return fail(IG_EINVAL, "n_up=%d outside 0..%d", d->n_up, IG_MAX_UP);
    int e;
    if ((e = check_conv_w(d->conv_in, "conv_in", 3))) return e;
    if (d->conv_in.cin != d->zc) return fail(IG_EINVAL, "conv_in takes %d channels, latent has %d", d->conv_in.cin, d->zc);
    int c = d->conv_in.cout, cp = d->conv_in.cout_p;
    NormCfg nc;
    if (d->norm_kind == IG_NORM_GROUP) {
        if (d->norm_groups < 1 || d->norm_groups > 128) return fail(IG_EINVAL, "norm_groups=%d outside 1..128", d->norm_groups);
        if (!(d->norm_eps >= 0.f) || d->norm_eps > 1.f) return fail(IG_EINVAL, "norm_eps=%g", (double)d->norm_eps);
        nc.groups = d->norm_groups;
    } else if (d->norm_kind != IG_NORM_RMS) {
        return fail(IG_EINVAL, "norm_kind=%d", d->norm_kind);
    }
    if ((e = check_resnet(d->mid[0], "mid.0", c, cp, nc))) return e;
    const ig_attn_w &a = d->attn;
    if ((e = check_gamma(a.gamma, "attn"))) return e;
    const ig_conv_w *aw[4] = {&a.q, &a.k, &a.v, &a.proj};
    const char *an[4] = {"attn.q", "attn.k", "attn.v", "attn.proj"};
    if (cp != c || c % 64) return fail(IG_EUNSUPPORTED, "attention width %d must be unpadded and a multiple of 64", c);
    if ((e = check_gn_site(nc, a.beta, c, cp, "attn"))) return e;
    for (int i = 0; i < 4; ++i) {
        if ((e = check_conv_w(*aw[i], an[i], 1))) return e;
        if (aw[i]->cin != c || aw[i]->cout != c || aw[i]->cin_p != c || aw[i]->cout_p != c)
            return fail(IG_EINVAL, "%s must map %d -> %d unpadded", an[i], c, c);
    }
    if ((int64_t)h0 * w0 >= (1LL << 30)) return fail(IG_EUNSUPPORTED, "latent too large for the attention");
    if ((e = check_resnet(d->mid[1], "mid.1", c, cp, nc))) return e;
    int64_t H = h0, W = w0;
    for (int s = 0; s < d->n_up; ++s) {
        const ig_up_w &u = d->ups[s];
        if (u.n_res < 0 || u.n_res > IG_MAX_RES) return fail(IG_EINVAL, "ups[%d].n_res=%d", s, u.n_res);
        wd.cp_in[s] = cp;
        const int c_in = c;
        for (int r = 0; r < u.n_res; ++r) {
            char nm[32];
            snprintf(nm, sizeof nm, "ups.%d.res.%d", s, r);
            if ((e = check_resnet(u.res[r], nm, c, cp, nc))) return e;
        }
        if (u.has_up) {
            char nm[32];
            snprintf(nm, sizeof nm, "ups.%d.up", s);
            if ((e = check_conv_w(u.up, nm, 3))) return e;
            if (u.up.cin != c || u.up.cin_p != cp) return fail(IG_EINVAL, "%s: input %d, stream %d", nm, u.up.cin, c);
            if (u.dupup) {
                if (u.dupup_ft < 1 || u.dupup_ft > 16) return fail(IG_EINVAL, "ups[%d].dupup_ft=%d", s, u.dupup_ft);
                if ((4LL * u.dupup_ft * u.up.cout) % c_in)
                    return fail(IG_EUNSUPPORTED, "ups[%d]: DupUp needs %d * %d a multiple of the input's %d channels", s,
                                u.up.cout, 4 * u.dupup_ft, c_in);
            }
            H *= 2;
            W *= 2;
            if (H * W >= (1LL << 31)) return fail(IG_EUNSUPPORTED, "frame too large");
            c = u.up.cout;
            cp = u.up.cout_p;
        } else if (u.dupup) {
            return fail(IG_EINVAL, "ups[%d]: a DupUp shortcut without an upsample", s);
        }
        wd.cp_out[s] = cp;
    }
    if ((e = check_gamma(d->norm_out_gamma, "norm_out"))) return e;
    if (d->norm_out_c != c) return fail(IG_EINVAL, "norm_out has %d channels, stream %d", d->norm_out_c, c);
    if ((e = check_gn_site(nc, d->norm_out_beta, c, cp, "norm_out"))) return e;
    if ((e = check_conv_w(d->conv_out, "conv_out", 3))) return e;
    if (d->conv_out.cin != c || d->conv_out.cin_p != cp) return fail(IG_EINVAL, "conv_out input %d, stream %d", d->conv_out.cin, c);
    pl.H = (int)H;
    pl.W = (int)W;
    return IG_OK;
}

// Sizes of up blocks s0..s1-1 run on `rows` rows (of W columns) of block
// s0's input level; feed[i]: the rows block i feeds to its upsample (NULL:
// all). fin: the output stage follows. xmax: the stream's maximum.
void size_blocks(const ig_decoder &d, int s0, int s1, int rows, int W, const Span *feed, bool fin, int cp,
                 int64_t &xmax, Plan &pl)
{
    for (int s = s0; s < s1; ++s) {
        const ig_up_w &u = d.ups[s];
        const int64_t M = (int64_t)rows * W;
        upd(xmax, M * cp);
        if (u.has_up && u.dupup) upd(pl.max_cp, M * cp);
        for (int r = 0; r < u.n_res; ++r) {
            size_resnet(u.res[r], M, cp, xmax, pl);
            cp = u.res[r].c2.cout_p;
        }
        if (u.has_up) {
            const int fr = feed ? feed[s].rows() : rows;
            upd(pl.max_xn, (int64_t)fr * W * cp);
            // the last resnet's conv2 casts all its rows; else only the fed ones
            upd(pl.max_xg, (int64_t)(u.n_res > 0 ? rows : fr) * W * cp);
            rows = 2 * fr;
            W *= 2;
            cp = u.up.cout_p;
            upd(xmax, (int64_t)rows * W * cp);
        }
    }
    if (fin) {
        const int64_t M = (int64_t)rows * W;
        upd(pl.max_xn, M * cp);
        size_gn(M, cp, pl);
        if (d.conv_out.cout > 16) upd(pl.max_h, M * d.conv_out.cout_p);  // else straight to the frame
    }
}

void band_structure(const ig_decoder &d, int *n_res, int *has_up)
{
    for (int i = 0; i < d.n_up; ++i) {
        n_res[i] = d.ups[i].n_res;
        has_up[i] = d.ups[i].has_up;
    }
}

int make_plan(const ig_decoder *d, int h0, int w0, int q_chunk, int band_rows, int band_from, Plan &pl)
{
    Widths wd;
    int e = check_decoder(d, h0, w0, wd, pl);
    if (e) return e;
    if (d->norm_kind == IG_NORM_GROUP) {
        pl.gn_groups = d->norm_groups;
        pl.gn_eps = d->norm_eps;
        if (band_rows > 0 && band_from >= 0 && band_from < d->n_up)
            return fail(IG_EUNSUPPORTED, "GroupNorm's statistics span the frame: a GroupNorm decoder does not run in bands");
    }
    pl.s = (band_rows > 0 && band_from >= 0 && band_from < d->n_up) ? band_from : d->n_up;
    pl.band_rows = pl.s < d->n_up ? band_rows : 0;
    // conv_in, the mid block and its attention run on the latent grid
    int64_t M = (int64_t)h0 * w0;
    const int c = d->mid[0].c2.cout;
    upd(pl.max_xn, M * d->conv_in.cin_p);
    upd(pl.max_x, M * d->conv_in.cout_p);
    size_resnet(d->mid[0], M, d->conv_in.cout_p, pl.max_x, pl);
    pl.m = (int)M;
    pl.mp = (int)((M + 63) / 64 * 64);
    pl.C = c;
    pl.flash = q_chunk <= 0 && flash_supported(pl.m, pl.mp, c);
    pl.qc = q_chunk > 0 ? q_chunk : 16384;
    if (pl.qc > pl.m) pl.qc = pl.m;
    upd(pl.max_xn, (int64_t)pl.mp * c);
    size_gn(pl.m, c, pl);
    if (!pl.flash && (uint64_t)pl.qc * pl.mp * 2 >= (3ULL << 30))
        return fail(IG_EUNSUPPORTED, "query chunk %d x %d keys: probabilities exceed 3 GiB; pass a smaller q_chunk", pl.qc, pl.mp);
    size_resnet(d->mid[1], M, c, pl.max_x, pl);
    // up blocks 0..s-1 on the whole frame (and the output when no bands)
    int lv = 0;
    for (int i = 0; i < pl.s; ++i) lv += d->ups[i].has_up ? 1 : 0;
    size_blocks(*d, 0, pl.s, h0, w0, nullptr, pl.s == d->n_up, d->mid[1].c2.cout_p, pl.max_x, pl);
    if (pl.s < d->n_up) {
        // every band from block s on; bands of band_rows kept output rows
        int n_res[IG_MAX_UP], has_up[IG_MAX_UP];
        band_structure(*d, n_res, has_up);
        for (int k0 = 0; k0 < pl.H; k0 += pl.band_rows) {
            const Span keep{k0, k0 + pl.band_rows < pl.H ? k0 + pl.band_rows : pl.H};
            Span input, feed[IG_MAX_UP];
            plan_band(d->n_up, n_res, has_up, h0, pl.s, keep, input, feed);
            size_blocks(*d, pl.s, d->n_up, input.rows(), w0 << lv, feed, true, wd.cp_in[pl.s], pl.max_xb, pl);
        }
    }
    // every 3x3 conv reads its f16 input from xn or xg
    if ((pl.max_xn > pl.max_xg ? pl.max_xn : pl.max_xg) * 2 >= kConvInMaxBytes)
        return fail(IG_EUNSUPPORTED, "a conv input of this frame passes %lld bytes; decode it in bands",
                    (long long)kConvInMaxBytes);
    // layout
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += round_up(bytes);
        return at;
    };
    const int64_t mp = pl.mp, C = pl.C, qc = pl.qc;
    pl.off_x = take(pl.max_x * 4);
    pl.off_xb = take(pl.max_xb * 4);
    pl.off_h = take(pl.max_h * 4);
    pl.off_xn = take(pl.max_xn * 2);
    pl.off_xg = take(pl.max_xg * 2);
    pl.off_q = take(mp * C * 2);
    pl.off_k = take(mp * C * 2);
    pl.off_vt = take(C * mp * 2);
    pl.off_cp = take(pl.max_cp * 4);
    pl.off_gn = take(pl.max_gn);
    if (pl.gn_groups) {
        // partials of the convs that feed a GroupNorm (the output frame
        // has the most tiles), for the stream and for conv1's output
        pl.gn_part = (size_t)pl.gn_groups * conv_gn_chunks(kConv3x3, pl.H, pl.W) * 3 * sizeof(float);
        pl.off_gpx = take(pl.gn_part);
        pl.off_gph = take(pl.gn_part);
        pl.off_gtab = take((size_t)3 * kConvMaxChannels * sizeof(float));
    }
    if (pl.flash) {
        // the single-pass kernel's key-range partials (if any)
        pl.off_o = take(0);
        pl.off_s = take(flash_workspace_bytes(pl.m, pl.C));
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
    float *cpb = nullptr;  // an up stage's input, for its DupUp shortcut
    void *gnws = nullptr;  // GroupNorm's statistics
    // GroupNorm decoders: the statistics of x and of h as gathered by the
    // conv that last wrote them (chunk counts; 0 when x or h changed since
    // or the conv could not gather them), and the per-channel table
    float *gpx = nullptr, *gph = nullptr, *gtab = nullptr;
    int gpx_n = 0, gph_n = 0;

    // whether a conv of these widths can gather its output's GroupNorm
    // statistics for the next norm
    bool gn_gathers(const ig_conv_w &cw) const
    {
        return pl.gn_groups && conv_gn_stats_supported(cw.cout_p, cw.cout, pl.gn_groups);
    }
    // the norm of the stream x (no bias on read): from the statistics its
    // producer gathered when it did, else the two-pass norm
    void norm_x(int M, int cp, int c_real, const float *gamma, const float *beta, int silu, _Float16 *y)
    {
        if (gpx_n)
            launch_groupnorm_partials(x, M, cp, c_real, pl.gn_groups, gamma, beta, silu, pl.gn_eps, gpx, gpx_n, gtab,
                                      y, s);
        else
            norm(x, M, cp, c_real, nullptr, gamma, beta, silu, y);
    }

    // the decoder's norm of M pixels (+ bias on read, + SiLU) -> f16 y
    void norm(const float *in, int M, int cp, int c_real, const float *bias, const float *gamma, const float *beta,
              int silu, _Float16 *y)
    {
        if (pl.gn_groups)
            launch_groupnorm(in, M, cp, c_real, pl.gn_groups, bias, gamma, beta, silu, pl.gn_eps, gnws, y, s);
        else
            launch_rmsnorm(in, M, cp, c_real, bias, gamma, silu, kEps, y, s);
    }

    // returns the chunk count of the GroupNorm partials written to gpart
    // (0 without gpart)
    int conv(int mode, const _Float16 *in, int H, int W, const ig_conv_w &cw, const float *bias,
             float oscale, int acc, float *out, _Float16 *yg = nullptr, float *gpart = nullptr)
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
        if (yg) {
            // the guarded cast of the result instead of the result
            a.yg = yg;
            a.gscale = ldexpf(1.f, -g);
            a.write_out = 0;
        }
        int nch = 0;
        if (gpart) {
            nch = conv_gn_chunks(mode, H, W);
            a.gn_part = gpart;
            a.gn_cpg = cw.cout / pl.gn_groups;
            a.gn_creal = cw.cout;
            a.gn_nchunk = nch;
        }
        launch_igemm(mode, a, s);
        return nch;
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

    // Up blocks s0..s1-1 on the stream x holding rows cur (buffer row 0 =
    // cur.first) of W columns and padded width cp ([QI] `run_blocks`); feed[i]:
    // the rows block i feeds to its upsample (NULL: all). Returns through
    // cur, W, cp the rows the stream then holds; normed: the last up conv
    // emitted norm_out's f16 input of conv_out into xn.
    void blocks(const ig_decoder &d, int s0, int s1, const Span *feed, Span &cur, int &W, int &cp, bool &normed)
    {
        const float gs = ldexpf(1.f, g);
        normed = false;
        for (int st = s0; st < s1; ++st) {
            const ig_up_w &u = d.ups[st];
            // the stage's input, for its DupUp shortcut (its real channels
            // decide the repeats)
            const int cp0 = cp, c0 = u.n_res > 0 ? u.res[0].c1.cin : u.up.cin;
            const bool dup = u.has_up && u.dupup;
            if (dup)
                (void)hipMemcpyAsync(cpb, x, (size_t)cur.rows() * W * cp * sizeof(float), hipMemcpyDeviceToDevice, s);
            for (int k = 0; k < u.n_res; ++k) {
                // a stage's last resnet before its up conv emits the
                // guarded cast itself
                const bool last = u.has_up && k == u.n_res - 1;
                resnet(u.res[k], cur.rows(), W, cp, last ? xg : nullptr);
                cp = u.res[k].c2.cout_p;
            }
            if (u.has_up) {
                const Span f = feed ? feed[st] : cur;
                const int64_t skip = (int64_t)(f.first - cur.first) * W;
                const _Float16 *up_in = xg + skip * cp;
                if (u.n_res == 0) {
                    launch_guard_cast(x + skip * cp, f.rows() * W, cp, nullptr, g, xg, s);
                    up_in = xg;
                }
                if (st == d.n_up - 1 && fusable(u.up) && d.norm_out_c == u.up.cout && !dup && !pl.gn_groups) {
                    // the last up conv's epilogue applies norm_out + SiLU; the
                    // f32 stream is not needed after it
                    conv_norm(kConv3x3Up2, up_in, f.rows(), W, u.up, u.up.b, gs, d.norm_out_gamma, d.norm_out_c, xn);
                    normed = true;
                } else {
                    gpx_n = conv(kConv3x3Up2, up_in, f.rows(), W, u.up, u.up.b, gs, 0, x, nullptr,
                                 gn_gathers(u.up) && !dup ? gpx : nullptr);
                }
                if (dup) {
                    gpx_n = 0;
                    // x[2y + sy][2x + sx] += the shuffled channels of the
                    // input's row y (the fed rows of the saved input)
                    const int factor = 4 * u.dupup_ft, repeats = u.up.cout * factor / c0;
                    launch_dupup(cpb + skip * cp0, f.rows(), W, cp0, x, u.up.cout, u.up.cout_p, factor, repeats,
                                 u.dupup_ft, s);
                }
                cur = Span{2 * f.first, 2 * f.end};
                W *= 2;
                cp = u.up.cout_p;
            }
        }
    }

    // norm_out + SiLU (unless fused), conv_out on the rows cur of the output
    // level (W columns), the rows keep of them into the NCHW frame of Hf
    // rows ([QI] `output_rows`)
    void output(const ig_decoder &d, Span cur, int W, int cp, bool normed, Span keep, int Hf, float *out)
    {
        const int H = cur.rows();
        if (!normed) norm_x(H * W, cp, d.norm_out_c, d.norm_out_gamma, d.norm_out_beta, 1, xn);
        float *o = out + (int64_t)cur.first * W;
        const int64_t plane = (int64_t)Hf * W;
        if (d.conv_out.cout <= 16) {
            // few output channels: straight into the NCHW frame
            launch_conv_out(xn, H, W, d.conv_out.cin_p, reinterpret_cast<const _Float16 *>(d.conv_out.w),
                            d.conv_out.cout, d.conv_out.cout_p, d.conv_out.b, o, s, keep.first - cur.first,
                            keep.end - cur.first, plane);
        } else {
            conv(kConv3x3, xn, H, W, d.conv_out, d.conv_out.b, 1.f, 0, h);
            const int64_t r0 = (int64_t)(keep.first - cur.first) * W;
            launch_nhwc_to_nchw(h + r0 * d.conv_out.cout_p, keep.rows() * W, d.conv_out.cout_p, d.conv_out.cout,
                                nullptr, out + (int64_t)keep.first * W, s, plane);
        }
    }

    // Rec::resnet with the combines folded into the epilogues; with cast,
    // conv2's epilogue emits the guarded f16 cast of the new stream into
    // cast instead of the stream itself (the stage's up conv reads only that)
    void resnet(const ig_resnet_w &r, int H, int W, int cp, _Float16 *cast = nullptr)
    {
        const int M = H * W;
        if (r.has_sc && !pl.gn_groups) {
            // one read of the stream gives the norm and the shortcut's
            // guarded input
            launch_rmsnorm(x, M, cp, r.c1.cin, nullptr, r.g1, 1, kEps, xn, s, xg, g);
            conv(kGemm, xg, H, W, r.sc, r.sc.b, ldexpf(1.f, g), 0, x);
        } else {
            norm_x(M, cp, r.c1.cin, r.g1, r.beta1, 1, xn);
            if (r.has_sc) {
                launch_guard_cast(x, M, cp, nullptr, g, xg, s);
                conv(kGemm, xg, H, W, r.sc, r.sc.b, ldexpf(1.f, g), 0, x);
                gpx_n = 0;
            }
        }
        // conv2 adds into the stream; with a GroupNorm next it gathers the
        // new stream's statistics (not when it emits only the guarded cast)
        float *g2 = (gn_gathers(r.c2) && !cast) ? gpx : nullptr;
        if (fusable(r.c1) && !pl.gn_groups) {
            // conv1's epilogue normalises (h + b1) itself; the f16 result
            // goes to the h region (conv1 still reads xn)
            _Float16 *hn = reinterpret_cast<_Float16 *>(h);
            conv_norm(kConv3x3, xn, H, W, r.c1, r.c1.b, 1.f, r.g2, r.c1.cout, hn);
            gpx_n = conv(kConv3x3, hn, H, W, r.c2, r.c2.b, 1.f, 1, x, cast, g2);
        } else if (gn_gathers(r.c1)) {
            // GroupNorm of (h + b1) from conv1's own statistics: conv1 adds
            // b1 in its epilogue (the same f32 sum the norm would form on
            // read) and gathers the statistics of what it stores
            gph_n = conv(kConv3x3, xn, H, W, r.c1, r.c1.b, 1.f, 0, h, nullptr, gph);
            launch_groupnorm_partials(h, M, r.c1.cout_p, r.c1.cout, pl.gn_groups, r.g2, r.beta2, 1, pl.gn_eps, gph,
                                      gph_n, gtab, xn, s);
            gpx_n = conv(kConv3x3, xn, H, W, r.c2, r.c2.b, 1.f, 1, x, cast, g2);
        } else {
            conv(kConv3x3, xn, H, W, r.c1, nullptr, 1.f, 0, h);
            norm(h, M, r.c1.cout_p, r.c1.cout, r.c1.b, r.g2, r.beta2, 1, xn);
            gpx_n = conv(kConv3x3, xn, H, W, r.c2, r.c2.b, 1.f, 1, x, cast, g2);
        }
    }

    // the mid attention, single head over the m latent pixels
    void attention(const ig_attn_w &a)
    {
        const int m = pl.m, mp = pl.mp, C = pl.C, qc = pl.qc;
        norm_x(m, C, C, a.gamma, a.beta, 0, xn);
        gpx_n = 0;  // the projection adds into the stream
        launch_zero_rows_f16(xn, m, mp, C, s);
        const _Float16 *wq = reinterpret_cast<const _Float16 *>(a.q.w);
        const _Float16 *wk = reinterpret_cast<const _Float16 *>(a.k.w);
        const _Float16 *wv = reinterpret_cast<const _Float16 *>(a.v.w);
        const _Float16 *wp = reinterpret_cast<const _Float16 *>(a.proj.w);
        // Q and K share xn: one launch covers both when the widths allow
        Gemm2Args qk{};
        qk.a = xn;
        qk.b = wq;
        qk.c = q16;
        qk.bias = a.q.b;
        qk.b2 = wk;
        qk.c2 = k16;
        qk.bias2 = a.k.b;
        qk.nsplit = C;
        qk.M = mp;
        qk.N = 2 * C;
        qk.K = C;
        qk.lda = C;
        qk.ldb = C;
        qk.ldc = C;
        qk.oscale = 1.f;
        if (gemm2_supported(qk)) {
            launch_gemm2(kEpiF16, qk, s);
        } else {
            gemm(xn, mp, C, C, wq, C, C, a.q.b, 1.f, q16, C, 1, 0);
            gemm(xn, mp, C, C, wk, C, C, a.k.b, 1.f, k16, C, 1, 0);
        }
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
            f.c = C;
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

namespace {

int run_decoder(const ig_decoder *dec, const float *latent, int h0, int w0, int guard_log2, int q_chunk,
                int band_rows, int band_from, void *ws, size_t ws_bytes, float *out, void *stream)
{
    clear_error();
    Plan pl;
    int e = make_plan(dec, h0, w0, q_chunk, band_rows, band_from, pl);
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
    r.cpb = reinterpret_cast<float *>(w + pl.off_cp);
    r.gnws = w + pl.off_gn;
    if (pl.gn_groups) {
        r.gpx = reinterpret_cast<float *>(w + pl.off_gpx);
        r.gph = reinterpret_cast<float *>(w + pl.off_gph);
        r.gtab = reinterpret_cast<float *>(w + pl.off_gtab);
    }
    hipStream_t s = r.s;
    (void)hipGetLastError();
    // latent -> f16 NHWC -> conv_in, x = conv + b
    launch_latent_ingest(latent, d.zc, h0 * w0, d.conv_in.cin_p, r.xn, s);
    r.gpx_n = r.conv(kConv3x3, r.xn, h0, w0, d.conv_in, d.conv_in.b, 1.f, 0, r.x, nullptr,
                     r.gn_gathers(d.conv_in) ? r.gpx : nullptr);
    r.resnet(d.mid[0], h0, w0, d.conv_in.cout_p);
    r.attention(d.attn);
    r.resnet(d.mid[1], h0, w0, d.mid[0].c2.cout_p);
    // up blocks 0..s-1 on the whole frame
    Span cur{0, h0};
    int W = w0, cp = d.mid[1].c2.cout_p;
    bool normed = false;
    r.blocks(d, 0, pl.s, nullptr, cur, W, cp, normed);
    if (pl.s == d.n_up) {
        r.output(d, cur, W, cp, normed, Span{0, pl.H}, pl.H, out);
        return check_launch("decoder_forward");
    }
    // the bands: blocks s.. from the saved whole-frame stream, each band's
    // input rows copied into its own stream buffer
    int n_res[IG_MAX_UP], has_up[IG_MAX_UP];
    band_structure(d, n_res, has_up);
    Run rb = r;
    rb.x = reinterpret_cast<float *>(w + pl.off_xb);
    for (int k0 = 0; k0 < pl.H; k0 += pl.band_rows) {
        const Span keep{k0, k0 + pl.band_rows < pl.H ? k0 + pl.band_rows : pl.H};
        Span input, feed[IG_MAX_UP];
        plan_band(d.n_up, n_res, has_up, h0, pl.s, keep, input, feed);
        const size_t row_bytes = (size_t)W * cp * sizeof(float);
        if (hipMemcpyAsync(rb.x, r.x + (int64_t)input.first * W * cp, row_bytes * input.rows(), hipMemcpyDeviceToDevice,
                           s) != hipSuccess)
            return fail(IG_EHIP, "band copy failed");
        Span bcur = input;
        int bW = W, bcp = cp;
        bool bnormed = false;
        rb.blocks(d, pl.s, d.n_up, feed, bcur, bW, bcp, bnormed);
        rb.output(d, bcur, bW, bcp, bnormed, keep, pl.H, out);
    }
    return check_launch("decoder_forward_bands");
}

}  // namespace

extern "C" {

size_t ig_decoder_workspace_bytes(const ig_decoder *dec, int h0, int w0, int q_chunk)
{
    clear_error();
    Plan pl;
    if (make_plan(dec, h0, w0, q_chunk, 0, 0, pl)) return 0;
    return pl.total;
}

int decoder_forward(const ig_decoder *dec, const float *latent, int h0, int w0, int guard_log2,
                    int q_chunk, void *ws, size_t ws_bytes, float *out, void *stream)
{
    return run_decoder(dec, latent, h0, w0, guard_log2, q_chunk, 0, 0, ws, ws_bytes, out, stream);
}

size_t ig_decoder_bands_workspace_bytes(const ig_decoder *dec, int h0, int w0, int q_chunk, int band_rows,
                                        int band_from)
{
    clear_error();
    Plan pl;
    if (make_plan(dec, h0, w0, q_chunk, band_rows, band_from, pl)) return 0;
    return pl.total;
}

int decoder_forward_bands(const ig_decoder *dec, const float *latent, int h0, int w0, int guard_log2,
                          int q_chunk, int band_rows, int band_from, void *ws, size_t ws_bytes, float *out,
                          void *stream)
{
    return run_decoder(dec, latent, h0, w0, guard_log2, q_chunk, band_rows, band_from, ws, ws_bytes, out,
                       stream);
}

int ig_band_plan(int n_up, const int *n_res, const int *has_up, int h0, int band_from, int keep_lo,
                 int keep_hi, int *input, int *feed)
{
    clear_error();
    if (n_up < 0 || n_up > IG_MAX_UP || h0 <= 0 || !n_res || !has_up || !input || (n_up > 0 && !feed))
        return fail(IG_EINVAL, "bad band plan arguments");
    if (band_from < 0 || band_from > n_up) return fail(IG_EINVAL, "band_from=%d outside 0..%d", band_from, n_up);
    int ups = 0;
    for (int i = 0; i < n_up; ++i) {
        if (n_res[i] < 0 || n_res[i] > IG_MAX_RES) return fail(IG_EINVAL, "n_res[%d]=%d", i, n_res[i]);
        ups += has_up[i] ? 1 : 0;
    }
    if (ups >= 24 || ((int64_t)h0 << ups) >= (1LL << 30)) return fail(IG_EINVAL, "frame too tall");
    const int hf = h0 << ups;
    if (keep_lo < 0 || keep_hi > hf || keep_lo >= keep_hi) return fail(IG_EINVAL, "keep rows [%d, %d) outside [0, %d)", keep_lo, keep_hi, hf);
    Span in, fd[IG_MAX_UP];
    plan_band(n_up, n_res, has_up, h0, band_from, Span{keep_lo, keep_hi}, in, fd);
    input[0] = in.first;
    input[1] = in.end;
    for (int i = 0; i < n_up; ++i) {
        feed[2 * i] = i >= band_from ? fd[i].first : 0;
        feed[2 * i + 1] = i >= band_from ? fd[i].end : 0;
    }
    return IG_OK;
}

}  // extern "C"
