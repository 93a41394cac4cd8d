// GroupNorm of the NHWC f32 stream into the next conv's f16 input, the norm
// of FLUX-class decoders (page "cortiq-engine 0.7.6, src/vae.rs",
// `GroupNorm::apply`: per group of channels, over all pixels, mean and
// population variance, y = (v - mean) / sqrt(var + eps) * gamma + beta;
// page "cortiq-engine 0.8.72, src/gpu_wgpu/s2v_vae.rs", GN_PART_SRC /
// GN_FIN_SRC / GN_APPLY_SRC and `gn`: bias on read, optional SiLU, f16 out).
//
// The pages reduce in two passes over memory (the sum, then the sum of
// squared deviations). Here one pass suffices: each workgroup holds a chunk
// of rows in registers, takes the chunk's per-group mean and then the
// squared deviations from it (the two-pass formula, from registers), and
// writes (count, mean, M2); a second kernel merges the chunks of a group
// pairwise in f64 (Chan, Golub and LeVeque's update:
// M2 = M2a + M2b + d^2 na nb / n, d = mean_b - mean_a), which is exact up
// to rounding for any chunking; the apply kernel reads the stream once more.
// HBM: two reads of the f32 stream and one f16 write.
#include "ig_internal.h"

namespace ig {
namespace {

constexpr int RPT = 8;          // rows per thread in a stats chunk
constexpr int MAXT = 256;       // threads per stats workgroup (at most)
constexpr int MAXG = 128;       // groups

__device__ __forceinline__ float silu1(float y) { return y / (1.0f + __expf(-y)); }

// one workgroup per chunk of RL * RPT rows; thread (rl, q): channel quad q,
// rows r0 + rl + RL k
__global__ void k_gn_stats(const float *__restrict__ x, int M, int cp, int c_real, int cpg, int groups,
                           const float *__restrict__ bias, float *__restrict__ part)
{
    __shared__ float ch_sum[MAXT * 4 / 1];  // per thread, reduced below
    __shared__ float g_mean[MAXG];
    const int nq = cp / 4;
    const int RL = blockDim.x / nq;
    const int t = threadIdx.x, q = t % nq, rl = t / nq;
    const int rows = RL * RPT;
    const int64_t r0 = (int64_t)blockIdx.x * rows;
    float4 v[RPT];
    bool ok[RPT];
    float4 b = {0.f, 0.f, 0.f, 0.f};
    if (bias) b = reinterpret_cast<const float4 *>(bias)[q];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int64_t r = r0 + rl + (int64_t)RL * k;
        ok[k] = r < M;
        if (ok[k]) {
            v[k] = reinterpret_cast<const float4 *>(x + r * cp)[q];
            v[k].x += b.x;
            v[k].y += b.y;
            v[k].z += b.z;
            v[k].w += b.w;
        } else {
            v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    int nrows = M - (int)r0;
    if (nrows > rows) nrows = rows;
    // pass 1 (registers): per-channel sums -> per-group means
    float4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        s.x += v[k].x;
        s.y += v[k].y;
        s.z += v[k].z;
        s.w += v[k].w;
    }
    float *cs = ch_sum;  // [RL][cp]
    cs[rl * cp + 4 * q + 0] = s.x;
    cs[rl * cp + 4 * q + 1] = s.y;
    cs[rl * cp + 4 * q + 2] = s.z;
    cs[rl * cp + 4 * q + 3] = s.w;
    __syncthreads();
    if (t < groups) {
        float a = 0.f;
        for (int c = t * cpg; c < (t + 1) * cpg; ++c)
            for (int l = 0; l < RL; ++l) a += cs[l * cp + c];
        g_mean[t] = a / (float)(nrows * cpg);
    }
    __syncthreads();
    // pass 2 (registers): squared deviations from the chunk's group mean
    float d2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = 4 * q + e;
        if (c >= c_real) continue;
        const float m = g_mean[c / cpg];
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            if (!ok[k]) continue;
            const float val = e == 0 ? v[k].x : e == 1 ? v[k].y : e == 2 ? v[k].z : v[k].w;
            const float d = val - m;
            d2[e] += d * d;
        }
    }
    cs[rl * cp + 4 * q + 0] = d2[0];
    cs[rl * cp + 4 * q + 1] = d2[1];
    cs[rl * cp + 4 * q + 2] = d2[2];
    cs[rl * cp + 4 * q + 3] = d2[3];
    __syncthreads();
    if (t < groups) {
        float a = 0.f;
        for (int c = t * cpg; c < (t + 1) * cpg; ++c)
            for (int l = 0; l < RL; ++l) a += cs[l * cp + c];
        float *o = part + ((int64_t)t * gridDim.x + blockIdx.x) * 3;  // [group][chunk][3]
        o[0] = (float)(nrows * cpg);
        o[1] = g_mean[t];
        o[2] = a;
    }
}

// one workgroup per group: merge its chunks' (n, mean, M2) in f64 and write
// (mean, 1 / sqrt(var + eps))
__global__ __launch_bounds__(256) void k_gn_final(const float *__restrict__ part, int nchunk, int groups,
                                                  float eps, float *__restrict__ stat)
{
    __shared__ double sn[256], sm[256], s2[256];
    const int g = blockIdx.x, t = threadIdx.x;
    double n = 0.0, m = 0.0, m2 = 0.0;
    for (int i = t; i < nchunk; i += 256) {
        const float *o = part + ((int64_t)g * nchunk + i) * 3;
        const double nb = o[0], mb = o[1], m2b = o[2];
        if (nb <= 0.0) continue;
        const double nn = n + nb, d = mb - m;
        m += d * nb / nn;
        m2 += m2b + d * d * n * nb / nn;
        n = nn;
    }
    sn[t] = n;
    sm[t] = m;
    s2[t] = m2;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (t < st) {
            const double na = sn[t], nb = sn[t + st];
            if (nb > 0.0) {
                const double nn = na + nb, d = sm[t + st] - sm[t];
                sm[t] += d * nb / nn;
                s2[t] += s2[t + st] + d * d * na * nb / nn;
                sn[t] = nn;
            }
        }
        __syncthreads();
    }
    if (t == 0) {
        const double var = sn[0] > 0.0 ? s2[0] / sn[0] : 0.0;
        stat[2 * g] = (float)sm[0];
        stat[2 * g + 1] = (float)(1.0 / sqrt(var + (double)eps));
    }
}

// y = ((x + b) - mean) * inv * gamma + beta (+ SiLU), f16; pad channels 0.
// Thread (rl, q) keeps channel quad q (its bias, gamma, beta and group
// statistics in registers) and walks rows rl, rl + RL, ...
__global__ __launch_bounds__(256) void k_gn_apply(const float *__restrict__ x, int M, int cp, int c_real, int cpg,
                                                  const float *__restrict__ bias, const float *__restrict__ stat,
                                                  const float *__restrict__ gamma, const float *__restrict__ beta,
                                                  int silu, _Float16 *__restrict__ y)
{
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const int nq = cp / 4;
    const int RL = blockDim.x / nq;
    const int q = threadIdx.x % nq, rl = threadIdx.x / nq;
    float b[4] = {0.f, 0.f, 0.f, 0.f}, sc[4], sh[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = 4 * q + e;
        if (bias) b[e] = bias[c];
        if (c < c_real) {
            const int g = c / cpg;
            // y = v * sc + sh with sc = inv * gamma, sh = beta - mean * inv * gamma
            sc[e] = stat[2 * g + 1] * gamma[c];
            sh[e] = beta[c] - stat[2 * g] * sc[e];
        } else {
            sc[e] = 0.f;
            sh[e] = 0.f;
        }
    }
    for (int64_t r = (int64_t)blockIdx.x * RL + rl; r < M; r += (int64_t)gridDim.x * RL) {
        const float4 v = reinterpret_cast<const float4 *>(x + r * cp)[q];
        const float vv[4] = {v.x, v.y, v.z, v.w};
        half4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float o = (vv[e] + b[e]) * sc[e] + sh[e];
            if (silu) o = silu1(o);
            h[e] = (_Float16)o;
        }
        reinterpret_cast<half4 *>(y + r * cp)[q] = h;
    }
}

int stats_threads(int cp)
{
    const int nq = cp / 4;
    const int rl = MAXT / nq;
    return nq * (rl > 0 ? rl : 1);
}

}  // namespace

int64_t gn_chunks(int M, int cp)
{
    const int rows = (stats_threads(cp) / (cp / 4)) * RPT;
    return ((int64_t)M + rows - 1) / rows;
}

size_t gn_workspace_bytes(int M, int cp, int groups)
{
    return (size_t)gn_chunks(M, cp) * groups * 3 * sizeof(float) + (size_t)groups * 2 * sizeof(float) + 256;
}

bool gn_supported(int cp, int c_real, int groups)
{
    return cp % 4 == 0 && cp / 4 <= MAXT && groups >= 1 && groups <= MAXG && c_real % groups == 0 &&
           c_real <= cp;
}

void launch_groupnorm(const float *x, int M, int cp, int c_real, int groups, const float *bias,
                      const float *gamma, const float *beta, int silu, float eps, void *ws, _Float16 *y,
                      hipStream_t s)
{
    if (M <= 0) return;
    const int nt = stats_threads(cp);
    const int64_t nchunk = gn_chunks(M, cp);
    float *part = reinterpret_cast<float *>(ws);
    float *stat = part + nchunk * groups * 3;
    const int cpg = c_real / groups;
    hipLaunchKernelGGL(k_gn_stats, dim3((unsigned)nchunk), dim3(nt), 0, s, x, M, cp, c_real, cpg, groups, bias, part);
    hipLaunchKernelGGL(k_gn_final, dim3(groups), dim3(256), 0, s, part, (int)nchunk, groups, eps, stat);
    const int rl = nt / (cp / 4);
    int64_t blocks = ((int64_t)M + rl - 1) / rl;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_gn_apply, dim3((unsigned)blocks), dim3(nt), 0, s, x, M, cp, c_real, cpg, bias, stat, gamma,
                       beta, silu, y);
}

}  // namespace ig
