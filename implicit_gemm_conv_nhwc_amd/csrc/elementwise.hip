// Memory-bound kernels of the decoder path on gfx950: the fused per-pixel
// RMS_norm, the range-guarded f16 cast, the residual combine, the attention
// softmax, latent ingest, the NCHW output, weight packing and a fill.
//
// Page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs": RMSN_SRC (norm with
// bias on read and optional SiLU, f16 out), CAST_SRC and `guard` (the
// guarded cast), `Rec::combine` (residual modes), `attention` (softmax of
// S f32 into P f16), OUT_SRC (NHWC -> NCHW with bias), `qconv` (the
// (tap, channel) weight plane), `decode` (latent ingest).
//
// These kernels are HBM-bound. They move 16-byte vectors per lane (float4
// in, four halves out), keep a pixel's channels in registers so its row is
// read once, and reduce within 16-lane groups with cross-lane shuffles
// instead of the pages' LDS tree.
#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4 to_half4(float4 v)
{
    half4 h;
    h[0] = (_Float16)v.x;
    h[1] = (_Float16)v.y;
    h[2] = (_Float16)v.z;
    h[3] = (_Float16)v.w;
    return h;
}

// SiLU, y / (1 + exp(-y)), with the hardware reciprocal (~1 ulp) in place of
// a full-precision divide (about ten instructions)
__device__ __forceinline__ float silu1(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// ---------------------------------------------------------------------
// RMS_norm: 16 lanes per pixel, each lane NCH float4 chunks (channels
// 4*(g + 16k) .. +3), so a wave handles 4 pixels and every load
// instruction reads 256 contiguous bytes per pixel; the row's bias and
// gamma come from LDS, staged once per workgroup. With yg, the same read
// also yields the guarded cast f16((x + b) * gscale) of the row (a resnet
// whose shortcut takes the raw stream), saving that cast's own read.
// ---------------------------------------------------------------------
template <int NCH>
__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ x, int M, int cp,
                                                 float sqrt_c, const float *__restrict__ bias,
                                                 const float *__restrict__ gamma, int silu,
                                                 float eps, _Float16 *__restrict__ y,
                                                 _Float16 *__restrict__ yg, float gscale)
{
    // the row's bias and gamma, staged once per workgroup: each lane then
    // reads its chunks from LDS instead of issuing 2 NCH vector loads
    __shared__ float4 s_b[16 * NCH], s_g[16 * NCH];
    for (int i = threadIdx.x; i < 16 * NCH; i += 256) {
        s_b[i] = bias ? reinterpret_cast<const float4 *>(bias)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        s_g[i] = reinterpret_cast<const float4 *>(gamma)[i];
    }
    const int g = threadIdx.x & 15;
    const int64_t pix = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    const bool live = pix < M;
    const float4 *xr = reinterpret_cast<const float4 *>(x + (live ? pix : 0) * cp);
    float4 v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) v[k] = xr[g + 16 * k];
    __syncthreads();
    if (!live) return;  // the 16 lanes of a pixel leave together
    if (bias) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const float4 b = s_b[g + 16 * k];
            v[k].x += b.x;
            v[k].y += b.y;
            v[k].z += b.z;
            v[k].w += b.w;
        }
    }
    if (yg) {
        half4 *gr = reinterpret_cast<half4 *>(yg + pix * cp);
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            gr[g + 16 * k] = to_half4(make_float4(v[k].x * gscale, v[k].y * gscale, v[k].z * gscale, v[k].w * gscale));
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    ss += __shfl_xor(ss, 8, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 1, 16);
    const float inv = sqrt_c / fmaxf(sqrtf(ss), eps);
    half4 *yr = reinterpret_cast<half4 *>(y + pix * cp);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const float4 gm = s_g[g + 16 * k];
        float4 o;
        o.x = v[k].x * inv * gm.x;
        o.y = v[k].y * inv * gm.y;
        o.z = v[k].z * inv * gm.z;
        o.w = v[k].w * inv * gm.w;
        if (silu) {
            o.x = silu1(o.x);
            o.y = silu1(o.y);
            o.z = silu1(o.z);
            o.w = silu1(o.w);
        }
        yr[g + 16 * k] = to_half4(o);
    }
}

// Rows of 768 or 1024 channels: one wave per pixel, lane g holding chunks
// g + 64 k, so every load instruction reads 1 KB of one row and the row is
// read once (the two-pass form below reads it twice; 1.8x faster at
// 65536 x 1024); the row's sum of squares reduces over the 64 lanes.
template <int NCH>
__global__ __launch_bounds__(256) void k_rmsnorm_row(const float *__restrict__ x, int M, int cp,
                                                     float sqrt_c, const float *__restrict__ bias,
                                                     const float *__restrict__ gamma, int silu,
                                                     float eps, _Float16 *__restrict__ y,
                                                     _Float16 *__restrict__ yg, float gscale)
{
    __shared__ float4 s_b[64 * NCH], s_g[64 * NCH];
    for (int i = threadIdx.x; i < 64 * NCH; i += 256) {
        s_b[i] = bias ? reinterpret_cast<const float4 *>(bias)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        s_g[i] = reinterpret_cast<const float4 *>(gamma)[i];
    }
    const int g = threadIdx.x & 63;
    const int64_t pix = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const bool live = pix < M;
    const float4 *xr = reinterpret_cast<const float4 *>(x + (live ? pix : 0) * cp);
    float4 v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) v[k] = xr[g + 64 * k];
    __syncthreads();
    if (!live) return;  // a pixel's wave leaves whole
    if (bias) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const float4 b = s_b[g + 64 * k];
            v[k].x += b.x;
            v[k].y += b.y;
            v[k].z += b.z;
            v[k].w += b.w;
        }
    }
    if (yg) {
        half4 *gr = reinterpret_cast<half4 *>(yg + pix * cp);
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            gr[g + 64 * k] = to_half4(make_float4(v[k].x * gscale, v[k].y * gscale, v[k].z * gscale, v[k].w * gscale));
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float inv = sqrt_c / fmaxf(sqrtf(ss), eps);
    half4 *yr = reinterpret_cast<half4 *>(y + pix * cp);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const float4 gm = s_g[g + 64 * k];
        float4 o;
        o.x = v[k].x * inv * gm.x;
        o.y = v[k].y * inv * gm.y;
        o.z = v[k].z * inv * gm.z;
        o.w = v[k].w * inv * gm.w;
        if (silu) {
            o.x = silu1(o.x);
            o.y = silu1(o.y);
            o.z = silu1(o.z);
            o.w = silu1(o.w);
        }
        yr[g + 64 * k] = to_half4(o);
    }
}

// Other rows wider than 512 channels: two passes over the pixel's row.
__global__ __launch_bounds__(256) void k_rmsnorm_wide(const float *__restrict__ x, int M, int cp,
                                                      float sqrt_c, const float *__restrict__ bias,
                                                      const float *__restrict__ gamma, int silu,
                                                      float eps, _Float16 *__restrict__ y,
                                                      _Float16 *__restrict__ yg, float gscale)
{
    const int g = threadIdx.x & 15;
    const int64_t pix = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (pix >= M) return;
    const float4 *xr = reinterpret_cast<const float4 *>(x + pix * cp);
    const float4 *b4 = reinterpret_cast<const float4 *>(bias);
    const int n4 = cp / 4;
    float ss = 0.f;
    for (int c = g; c < n4; c += 16) {
        float4 v = xr[c];
        if (bias) {
            const float4 b = b4[c];
            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
        }
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        if (yg)
            reinterpret_cast<half4 *>(yg + pix * cp)[c] =
                to_half4(make_float4(v.x * gscale, v.y * gscale, v.z * gscale, v.w * gscale));
    }
    ss += __shfl_xor(ss, 8, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 1, 16);
    const float inv = sqrt_c / fmaxf(sqrtf(ss), eps);
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
    half4 *yr = reinterpret_cast<half4 *>(y + pix * cp);
    for (int c = g; c < n4; c += 16) {
        float4 v = xr[c];
        if (bias) {
            const float4 b = b4[c];
            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
        }
        const float4 gm = g4[c];
        float4 o;
        o.x = v.x * inv * gm.x;
        o.y = v.y * inv * gm.y;
        o.z = v.z * inv * gm.z;
        o.w = v.w * inv * gm.w;
        if (silu) {
            o.x = silu1(o.x); o.y = silu1(o.y); o.z = silu1(o.z); o.w = silu1(o.w);
        }
        yr[c] = to_half4(o);
    }
}

// ---------------------------------------------------------------------
// guarded cast: y = f16((x + b) * 2^-g), one float4 per lane per step
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_guard_cast(const float *__restrict__ x, int64_t n4,
                                                    int C4, const float *__restrict__ bias,
                                                    float scale, _Float16 *__restrict__ y)
{
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const float4 *b4 = reinterpret_cast<const float4 *>(bias);
    half4 *y4 = reinterpret_cast<half4 *>(y);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * 256) {
        // the stream's last read before the conv that takes the cast (the
        // up conv writes a new stream): a streaming (nontemporal) load
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x4 + i));
        float4 v = make_float4(t[0], t[1], t[2], t[3]);
        if (bias) {
            const float4 b = b4[i % C4];
            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
        }
        v.x *= scale; v.y *= scale; v.z *= scale; v.w *= scale;
        y4[i] = to_half4(v);
    }
}

// ---------------------------------------------------------------------
// combine: t = h + hb is added into x (mode 0), replaces x together with
// the shortcut s + sb (mode 1), or replaces x alone (mode 2)
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(float *__restrict__ x, const float *__restrict__ h,
                                                 const float *__restrict__ hb,
                                                 const float *__restrict__ sv,
                                                 const float *__restrict__ sb, int64_t n4, int C4,
                                                 int mode)
{
    float4 *x4 = reinterpret_cast<float4 *>(x);
    const float4 *h4 = reinterpret_cast<const float4 *>(h);
    const float4 *s4 = reinterpret_cast<const float4 *>(sv);
    const float4 *hb4 = reinterpret_cast<const float4 *>(hb);
    const float4 *sb4 = reinterpret_cast<const float4 *>(sb);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * 256) {
        const int c = (int)(i % C4);
        float4 t = h4[i];
        if (hb) {
            const float4 b = hb4[c];
            t.x += b.x; t.y += b.y; t.z += b.z; t.w += b.w;
        }
        float4 base;
        if (mode == 0) {
            base = x4[i];
        } else if (mode == 1) {
            base = s4[i];
            if (sb) {
                const float4 b = sb4[c];
                base.x += b.x; base.y += b.y; base.z += b.z; base.w += b.w;
            }
        } else {
            base = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        base.x += t.x; base.y += t.y; base.z += t.z; base.w += t.w;
        x4[i] = base;
    }
}

// ---------------------------------------------------------------------
// row softmax S f32 -> P f16; one workgroup per row; online max/sum in one
// pass, then the normalised write
// ---------------------------------------------------------------------
__device__ __forceinline__ void ms_merge(float &m, float &s, float m2, float s2)
{
    if (m2 == -INFINITY) return;
    if (m == -INFINITY) {
        m = m2;
        s = s2;
        return;
    }
    const float mx = fmaxf(m, m2);
    s = s * __expf(m - mx) + s2 * __expf(m2 - mx);
    m = mx;
}

__global__ __launch_bounds__(256) void k_softmax(const float *__restrict__ S, int lds, int valid,
                                                 int ncols, _Float16 *__restrict__ P, int ldp)
{
    const int64_t row = blockIdx.x;
    const float *s = S + row * lds;
    _Float16 *pr = P + row * ldp;
    const int tid = threadIdx.x;
    float m = -INFINITY, sum = 0.f;
    const int v4 = valid >> 2;
    const float4 *s4 = reinterpret_cast<const float4 *>(s);
    for (int j = tid; j < v4; j += 256) {
        const float4 t = s4[j];
        const float mx = fmaxf(fmaxf(t.x, t.y), fmaxf(t.z, t.w));
        const float part = __expf(t.x - mx) + __expf(t.y - mx) + __expf(t.z - mx) + __expf(t.w - mx);
        ms_merge(m, sum, mx, part);
    }
    for (int j = 4 * v4 + tid; j < valid; j += 256) ms_merge(m, sum, s[j], 1.f);
    // wave reduce
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const float s2 = __shfl_xor(sum, off);
        ms_merge(m, sum, m2, s2);
    }
    __shared__ float red_m[4], red_s[4];
    if ((tid & 63) == 0) {
        red_m[tid >> 6] = m;
        red_s[tid >> 6] = sum;
    }
    __syncthreads();
    m = red_m[0];
    sum = red_s[0];
    for (int w = 1; w < 4; ++w) ms_merge(m, sum, red_m[w], red_s[w]);
    const float inv = 1.0f / sum;
    half4 *p4 = reinterpret_cast<half4 *>(pr);
    for (int j = tid; j < v4; j += 256) {
        const float4 t = s4[j];
        float4 o;
        o.x = __expf(t.x - m) * inv;
        o.y = __expf(t.y - m) * inv;
        o.z = __expf(t.z - m) * inv;
        o.w = __expf(t.w - m) * inv;
        p4[j] = to_half4(o);
    }
    for (int j = 4 * v4 + tid; j < ncols; j += 256)
        pr[j] = (j < valid) ? (_Float16)(__expf(s[j] - m) * inv) : (_Float16)0.f;
}

// ---------------------------------------------------------------------
// latent ingest: NCHW f32 [zc][M] -> NHWC f16 [M][cp], zero past zc
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_latent(const float *__restrict__ z, int zc, int M, int cp8,
                                                _Float16 *__restrict__ y)
{
    const int64_t n = (int64_t)M * cp8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t p = i / cp8;
        const int c0 = (int)(i - p * cp8) * 8;
        half8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            h[e] = (c0 + e < zc) ? (_Float16)z[(int64_t)(c0 + e) * M + p] : (_Float16)0.f;
        reinterpret_cast<half8 *>(y)[i] = h;
    }
}

// ---------------------------------------------------------------------
// output: NHWC f32 [M][ld] (first nch channels) + bias -> NCHW [nch][M]
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_out(const float *__restrict__ y, int M, int ld, int nch,
                                             const float *__restrict__ bias, float *__restrict__ out, int64_t HWo)
{
    for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < M; p += (int64_t)gridDim.x * 256)
        for (int ch = 0; ch < nch; ++ch)
            out[(int64_t)ch * HWo + p] = y[p * ld + ch] + (bias ? bias[ch] : 0.f);
}

// ---------------------------------------------------------------------
// weight planes from OIHW [cout][cin][k][k], zero padded: 1x1 ->
// [cout_p][cin_p] (the GEMM's B rows); 3x3 -> [cin_p/16][9][cout_p][16]
// (for each 16-channel slice and tap, the output channels' 16 weights are
// contiguous, so a conv stage reads its weights as one block)
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack(const _Float16 *__restrict__ w, int cout, int cin,
                                              int kk, int cout_p, int cin_p,
                                              _Float16 *__restrict__ plane)
{
    const int64_t n = (int64_t)cout_p * kk * cin_p;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        int ci, tap, o;
        if (kk == 1) {  // [cout_p][cin_p]
            ci = (int)(i % cin_p);
            o = (int)(i / cin_p);
            tap = 0;
        } else {  // [cin_p/16][9][cout_p][16]
            const int c16 = (int)(i & 15);
            const int64_t rest = i >> 4;
            o = (int)(rest % cout_p);
            tap = (int)((rest / cout_p) % kk);
            ci = (int)(rest / ((int64_t)cout_p * kk)) * 16 + c16;
        }
        plane[i] = (o < cout && ci < cin) ? w[((int64_t)o * cin + ci) * kk + tap] : (_Float16)0.f;
    }
}

// DupUp shortcut: the output pixel in corner q = 2 sy + sx of the 2x2 block
// over half-resolution pixel p gets, in output channel o, the value of p's
// channel (factor o + 4 (ft - 1) + q) / repeats (a channel-to-space shuffle
// of repeated channels). A thread owns one half-resolution pixel and four
// consecutive output channels, and updates the four corners of its block
// with one 16-byte read-add-write each; its source channels lie in the
// pixel's row of src, which the four corners share.
__global__ __launch_bounds__(256) void k_dupup(const float *__restrict__ src, int W, int cin_p,
                                               float *__restrict__ x, int cout, int cout_p,
                                               int factor, int repeats, int ft, int64_t n)
{
    const int q4 = cout_p / 4;  // channel quads per output pixel
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t p = i / q4;
        const int o0 = (int)(i - p * q4) * 4;
        if (o0 >= cout) continue;
        const int64_t y = p / W;
        const int xc = (int)(p - y * W);
        const float *row = src + p * cin_p;
        const int shift = 4 * (ft - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 add;
            float *a = &add.x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = o0 + e;
                a[e] = o < cout ? row[(factor * o + shift + q) / repeats] : 0.f;
            }
            const int64_t out_pix = (2 * y + (q >> 1)) * (2 * (int64_t)W) + 2 * xc + (q & 1);
            float4 *dst = reinterpret_cast<float4 *>(x + out_pix * cout_p + o0);
            float4 v = *dst;
            v.x += add.x;
            v.y += add.y;
            v.z += add.z;
            v.w += add.w;
            *dst = v;
        }
    }
}

__global__ __launch_bounds__(256) void k_zero_f16(_Float16 *__restrict__ y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        y[i] = (_Float16)0.f;
}

inline unsigned blocks_for(int64_t n, int64_t per = 256, int64_t cap = 1 << 20)
{
    int64_t b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (unsigned)b;
}

}  // namespace

void launch_rmsnorm(const float *x, int M, int cp, int c_real, const float *bias,
                    const float *gamma, int silu, float eps, _Float16 *y, hipStream_t s, _Float16 *yg,
                    int guard_log2)
{
    if (M <= 0) return;
    const float sqrt_c = sqrtf((float)c_real);
    const float gscale = ldexpf(1.0f, -guard_log2);
    if (cp == 768 || cp == 1024) {
        const unsigned grid_row = (unsigned)(((int64_t)M * 64 + 255) / 256);
        switch (cp / 256) {
#define IG_NORM_ROW_CASE(n)                                                                      \
    case n:                                                                                      \
        hipLaunchKernelGGL(k_rmsnorm_row<n>, dim3(grid_row), dim3(256), 0, s, x, M, cp, sqrt_c, \
                           bias, gamma, silu, eps, y, yg, gscale);                               \
        break;
            IG_NORM_ROW_CASE(3)
            IG_NORM_ROW_CASE(4)
#undef IG_NORM_ROW_CASE
        }
        return;
    }
    const unsigned grid = (unsigned)(((int64_t)M * 16 + 255) / 256);
    switch (cp / 64) {
#define IG_NORM_CASE(n)                                                                          \
    case n:                                                                                      \
        hipLaunchKernelGGL(k_rmsnorm<n>, dim3(grid), dim3(256), 0, s, x, M, cp, sqrt_c, bias,    \
                           gamma, silu, eps, y, yg, gscale);                                     \
        break;
        IG_NORM_CASE(1)
        IG_NORM_CASE(2)
        IG_NORM_CASE(3)
        IG_NORM_CASE(4)
        IG_NORM_CASE(5)
        IG_NORM_CASE(6)
        IG_NORM_CASE(7)
        IG_NORM_CASE(8)
#undef IG_NORM_CASE
    default:
        hipLaunchKernelGGL(k_rmsnorm_wide, dim3(grid), dim3(256), 0, s, x, M, cp, sqrt_c, bias,
                           gamma, silu, eps, y, yg, gscale);
    }
}

void launch_guard_cast(const float *x, int M, int C, const float *bias, int guard_log2,
                       _Float16 *y, hipStream_t s)
{
    const int64_t n4 = (int64_t)M * C / 4;
    if (n4 <= 0) return;
    const float scale = ldexpf(1.0f, -guard_log2);
    hipLaunchKernelGGL(k_guard_cast, dim3(blocks_for(n4, 256, 8192)), dim3(256), 0, s, x, n4, C / 4,
                       bias, scale, y);
}

void launch_combine(float *x, const float *h, const float *hb, const float *sv, const float *sb,
                    int M, int C, int mode, hipStream_t s)
{
    const int64_t n4 = (int64_t)M * C / 4;
    if (n4 <= 0) return;
    hipLaunchKernelGGL(k_combine, dim3(blocks_for(n4, 256, 8192)), dim3(256), 0, s, x, h, hb, sv, sb,
                       n4, C / 4, mode);
}

void launch_softmax(const float *S, int rows, int lds, int valid, int ncols, _Float16 *P, int ldp,
                    hipStream_t s)
{
    if (rows <= 0) return;
    hipLaunchKernelGGL(k_softmax, dim3(rows), dim3(256), 0, s, S, lds, valid, ncols, P, ldp);
}

void launch_latent_ingest(const float *z, int zc, int M, int cp, _Float16 *y, hipStream_t s)
{
    const int64_t n = (int64_t)M * (cp / 8);
    if (n <= 0) return;
    hipLaunchKernelGGL(k_latent, dim3(blocks_for(n, 256, 1 << 20)), dim3(256), 0, s, z, zc, M,
                       cp / 8, y);
}

void launch_nhwc_to_nchw(const float *y, int M, int ld, int nch, const float *bias, float *out,
                         hipStream_t s, int64_t HWo)
{
    if (M <= 0) return;
    hipLaunchKernelGGL(k_out, dim3(blocks_for(M, 256, 1 << 20)), dim3(256), 0, s, y, M, ld, nch,
                       bias, out, HWo > 0 ? HWo : (int64_t)M);
}

void launch_pack_weights(const _Float16 *w, int cout, int cin, int k, int cout_p, int cin_p,
                         _Float16 *plane, hipStream_t s)
{
    const int64_t n = (int64_t)cout_p * k * k * cin_p;
    hipLaunchKernelGGL(k_pack, dim3(blocks_for(n, 256, 1 << 20)), dim3(256), 0, s, w, cout, cin,
                       k * k, cout_p, cin_p, plane);
}

void launch_zero_rows_f16(_Float16 *y, int r0, int r1, int ld, hipStream_t s)
{
    const int64_t n = (int64_t)(r1 - r0) * ld;
    if (n <= 0) return;
    hipLaunchKernelGGL(k_zero_f16, dim3(blocks_for(n, 256, 1 << 20)), dim3(256), 0, s,
                       y + (int64_t)r0 * ld, n);
}

void launch_dupup(const float *src, int H, int W, int cin_p, float *x, int cout, int cout_p,
                  int factor, int repeats, int ft, hipStream_t s)
{
    const int64_t n = (int64_t)H * W * (cout_p / 4);
    if (n <= 0 || cout <= 0) return;
    hipLaunchKernelGGL(k_dupup, dim3(blocks_for(n, 256, 1 << 20)), dim3(256), 0, s, src, W, cin_p, x,
                       cout, cout_p, factor, repeats, ft, n);
}

}  // namespace ig
