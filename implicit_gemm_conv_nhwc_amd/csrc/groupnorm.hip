// GroupNorm of the NHWC f32 stream into the next conv's f16 input, the norm
// of FLUX-class decoders (page "cortiq-engine 0.7.6, src/vae.rs",
// `GroupNorm::apply`: per group of channels, over all pixels, mean and
// population variance, y = (v - mean) / sqrt(var + eps) * gamma + beta;
// page "cortiq-engine 0.8.72, src/gpu_wgpu/s2v_vae.rs", GN_PART_SRC /
// GN_FIN_SRC / GN_APPLY_SRC and `gn`: bias on read, optional SiLU, f16 out).
//
// The pages reduce in two passes over memory (the sum, then the sum of
// squared deviations). Here one pass suffices: a thread holds a batch of
// rows of its channel quad in registers, takes the batch's mean and the
// squared deviations from it (the two-pass formula, from registers), and
// folds them into running per-channel (count, mean, M2) with Chan, Golub
// and LeVeque's update (M2 = M2a + M2b + d^2 na nb / n, d = mean_b -
// mean_a), exact up to rounding for any split. Each of at most 1024
// workgroups merges its threads' figures per group and writes one partial;
// a second kernel merges a group's partials in f64 and turns the group
// statistics into a per-channel offset and scale; the apply kernel reads the
// stream once more. HBM: two reads of the f32 stream and one f16 write.
#include <mutex>

#include "ig_internal.h"

namespace ig {
namespace {

constexpr int RPT = 8;          // rows per thread in a batch
constexpr int MAXT = 256;       // threads per stats workgroup (at most)
constexpr int MAXG = 128;       // groups
constexpr int MAXCHUNK = 1024;  // stats workgroups, i.e. partials per group

typedef float f32x4 __attribute__((ext_vector_type(4)));

// SiLU, y / (1 + exp(-y)), with the hardware reciprocal (~1 ulp) in place of
// a full-precision divide (about ten instructions)
__device__ __forceinline__ float silu1(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// Chan, Golub and LeVeque's merge of (nb, mb, m2b) into (n, m, m2)
__device__ __forceinline__ void chan_merge(float &n, float &m, float &m2, float nb, float mb, float m2b)
{
    const float nn = n + nb, wb = nb / nn, d = mb - m;
    m += d * wb;
    m2 += m2b + d * d * n * wb;
    n = nn;
}

// Workgroup w walks the batches w, w + gridDim.x, ... of RL * RPT rows.
// Thread (rl, q) holds channel quad q of rows rl + RL k of a batch in
// registers, takes the batch's per-channel mean and squared deviations from
// it, and merges them into its running per-channel (count, mean, M2). At
// the end the workgroup merges its threads' per-channel figures into
// per-group ones and writes them as chunk w of each group.
__global__ __launch_bounds__(256) void k_gn_stats(const float *__restrict__ x, int M, int cp, int cpg, int groups,
                                                  const float *__restrict__ bias, int64_t nbatch,
                                                  float *__restrict__ part)
{
    __shared__ float s_mean[MAXT * 4], s_m2[MAXT * 4];  // [rl][cp]
    __shared__ float s_n[MAXT];                         // [rl]
    const int nq = cp / 4;
    const int RL = blockDim.x / nq;
    const int t = threadIdx.x, q = t % nq, rl = t / nq;
    const int rows = RL * RPT;
    const float4 b = bias ? reinterpret_cast<const float4 *>(bias)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    float n = 0.f, mean[4] = {0.f, 0.f, 0.f, 0.f}, m2[4] = {0.f, 0.f, 0.f, 0.f};
    // rows r0 + RL k of a batch grow with k: the valid ones are a prefix
    // (rows past the end load row M - 1, unused: no branch around a load,
    // so the compiler can keep the next batch's loads in flight)
    auto load = [&](int64_t bt, float4 *v) __attribute__((always_inline)) {
        const int64_t r0 = bt * rows + rl;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int64_t r = r0 + (int64_t)RL * k;
            // streaming (nontemporal) loads: measured faster here than loads
            // that leave the stream in the caches for the apply kernel's read
            const f32x4 u = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + (r < M ? r : (int64_t)M - 1) * cp) + q);
            v[k] = make_float4(u[0], u[1], u[2], u[3]);
        }
    };
    // fold batch bt (held in v) into the running figures
    auto fold = [&](int64_t bt, float4 *v) __attribute__((always_inline)) {
        int64_t left = (int64_t)M - (bt * rows + rl);  // rows of this lane still in range
        left = left < 0 ? 0 : (left > rows ? rows : left);
        const int nb = ((int)left + RL - 1) / RL;
        if (nb == 0) return;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            if (k < nb) {
                v[k].x += b.x;
                v[k].y += b.y;
                v[k].z += b.z;
                v[k].w += b.w;
            }
        }
        float bm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            if (k < nb) {
                bm[0] += v[k].x;
                bm[1] += v[k].y;
                bm[2] += v[k].z;
                bm[3] += v[k].w;
            }
        }
        const float inb = 1.f / (float)nb;
#pragma unroll
        for (int e = 0; e < 4; ++e) bm[e] *= inb;
        float bq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            if (k < nb) {
                const float d0 = v[k].x - bm[0], d1 = v[k].y - bm[1], d2 = v[k].z - bm[2], d3 = v[k].w - bm[3];
                bq[0] += d0 * d0;
                bq[1] += d1 * d1;
                bq[2] += d2 * d2;
                bq[3] += d3 * d3;
            }
        }
        const float nn = n + (float)nb, wb = (float)nb / nn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d = bm[e] - mean[e];
            mean[e] += d * wb;
            m2[e] += bq[e] + d * d * n * wb;
        }
        n = nn;
    };
    // two register sets in turn: one batch's loads are in flight while the
    // other is folded
    float4 v[RPT], w[RPT];
    const int64_t step = gridDim.x;
    load(blockIdx.x, v);
    for (int64_t bt = blockIdx.x; bt < nbatch; bt += 2 * step) {
        load(bt + step, w);
        fold(bt, v);
        load(bt + 2 * step, v);
        fold(bt + step, w);  // (a batch past the end folds nothing)
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        s_mean[rl * cp + 4 * q + e] = mean[e];
        s_m2[rl * cp + 4 * q + e] = m2[e];
    }
    if (q == 0) s_n[rl] = n;  // every quad of a row lane saw the same rows
    __syncthreads();
    if (t < groups) {
        float gn = 0.f, gm = 0.f, gq = 0.f;
        for (int l = 0; l < RL; ++l) {
            const float nl = s_n[l];
            if (nl <= 0.f) continue;
            for (int c = t * cpg; c < (t + 1) * cpg; ++c) chan_merge(gn, gm, gq, nl, s_mean[l * cp + c], s_m2[l * cp + c]);
        }
        float *o = part + ((int64_t)t * gridDim.x + blockIdx.x) * 3;  // [group][chunk][3]
        o[0] = gn;
        o[1] = gm;
        o[2] = gq;
    }
}

// one workgroup per group: merge its chunks' (n, mean, M2) in f64, then
// write the group's per-channel offset mean - b (in f64, rounded once),
// scale inv * gamma and beta (workgroup 0 also zeroes the pad channels')
__global__ __launch_bounds__(256) void k_gn_final(const float *__restrict__ part, int nchunk, int cp, int c_real,
                                                  int cpg, float eps, const float *__restrict__ bias,
                                                  const float *__restrict__ gamma, const float *__restrict__ beta,
                                                  float *__restrict__ off, float *__restrict__ sc,
                                                  float *__restrict__ sh)
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
    const double var = sn[0] > 0.0 ? s2[0] / sn[0] : 0.0;
    const float inv = (float)(1.0 / sqrt(var + (double)eps));
    for (int c = g * cpg + t; c < (g + 1) * cpg; c += 256) {
        // the statistics are of v = x + b: (v - mean) = x - (mean - b)
        off[c] = (float)(sm[0] - (bias ? (double)bias[c] : 0.0));
        sc[c] = inv * gamma[c];
        sh[c] = beta[c];
    }
    if (g == 0)
        for (int c = c_real + t; c < cp; c += 256) {
            off[c] = 0.f;
            sc[c] = 0.f;
            sh[c] = 0.f;
        }
}

// y = (x - off) * scale + beta (+ SiLU), f16, with the per-channel offset
// mean - b and scale inv * gamma: subtracting the mean first keeps the f32
// rounding to the mean's own (0 on pad channels).
// Workgroup w covers rows w RL AU .. (w + 1) RL AU - 1; thread (rl, q)
// issues the loads of its AU rows (channel quad q) first.
constexpr int AU = 2;  // rows per thread in the apply kernel
__global__ __launch_bounds__(256) void k_gn_apply(const float *__restrict__ x, int M, int cp,
                                                  const float *__restrict__ offset, const float *__restrict__ scale,
                                                  const float *__restrict__ shift, int silu, _Float16 *__restrict__ y)
{
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const int nq = cp / 4;
    const int RL = blockDim.x / nq;
    const int q = threadIdx.x % nq, rl = threadIdx.x / nq;
    const int64_t r0 = (int64_t)blockIdx.x * RL * AU + rl;
    f32x4 v[AU];
#pragma unroll
    for (int k = 0; k < AU; ++k) {
        const int64_t r = r0 + (int64_t)RL * k;
        // the stream's last read here: a streaming (nontemporal) load (rows
        // past the end load row M - 1 and are not written)
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + (r < M ? r : (int64_t)M - 1) * cp) + q);
    }
    // the per-channel offset, scale and shift, staged once per workgroup
    __shared__ float4 s_b[MAXT], s_a[MAXT], s_s[MAXT];
    for (int i = threadIdx.x; i < nq; i += blockDim.x) {
        s_b[i] = reinterpret_cast<const float4 *>(offset)[i];
        s_a[i] = reinterpret_cast<const float4 *>(scale)[i];
        s_s[i] = reinterpret_cast<const float4 *>(shift)[i];
    }
    __syncthreads();
    const float4 b = s_b[q], a4 = s_a[q], s4 = s_s[q];
    const float bb[4] = {b.x, b.y, b.z, b.w}, sc[4] = {a4.x, a4.y, a4.z, a4.w}, sh[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int k = 0; k < AU; ++k) {
        const int64_t r = r0 + (int64_t)RL * k;
        if (r >= M) break;
        half4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float o = (v[k][e] - bb[e]) * sc[e] + sh[e];
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
    const int64_t nbatch = ((int64_t)M + rows - 1) / rows;
    return nbatch < MAXCHUNK ? nbatch : MAXCHUNK;
}

size_t gn_workspace_bytes(int M, int cp, int groups)
{
    return ((size_t)gn_chunks(M, cp) * groups * 3 + (size_t)cp * 3) * sizeof(float) + 256;
}

// The allocation-free entry point's workspace: a file-scope device array
// sized for every supported call (at most MAXCHUNK partials per group, MAXG
// groups, 4 MAXT channels), one copy per GPU for the life of the process.
// Host code never passes its name to a kernel (on the host it only stands
// for the symbol): the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
constexpr size_t kGnScratchBytes = ((size_t)MAXCHUNK * MAXG * 3 + (size_t)MAXT * 4 * 3) * sizeof(float) + 256;
static __device__ __align__(256) char gn_scratch[kGnScratchBytes];

size_t gn_scratch_bytes() { return kGnScratchBytes; }

void *gn_scratch_ptr()
{
    constexpr int kMaxDev = 64;
    static void *ptr[kMaxDev] = {};
    static std::mutex mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(gn_scratch)) != hipSuccess || !p) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
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
    const int rows = (nt / (cp / 4)) * RPT;
    const int64_t nbatch = ((int64_t)M + rows - 1) / rows;
    float *part = reinterpret_cast<float *>(ws);
    // the per-channel table, 16-byte aligned for the apply kernel's vector
    // loads (cp is a multiple of 4; the workspace holds 256 bytes of slack)
    const uintptr_t tab = (reinterpret_cast<uintptr_t>(part + nchunk * groups * 3) + 15) & ~(uintptr_t)15;
    float *offset = reinterpret_cast<float *>(tab), *scale = offset + cp, *shift = scale + cp;
    const int cpg = c_real / groups;
    hipLaunchKernelGGL(k_gn_stats, dim3((unsigned)nchunk), dim3(nt), 0, s, x, M, cp, cpg, groups, bias, nbatch, part);
    hipLaunchKernelGGL(k_gn_final, dim3(groups), dim3(256), 0, s, part, (int)nchunk, cp, c_real, cpg, eps, bias, gamma,
                       beta, offset, scale, shift);
    const int rl = nt / (cp / 4);
    const int64_t blocks = ((int64_t)M + (int64_t)rl * AU - 1) / ((int64_t)rl * AU);
    hipLaunchKernelGGL(k_gn_apply, dim3((unsigned)blocks), dim3(nt), 0, s, x, M, cp, offset, scale, shift, silu, y);
}

// The statistics arrive as partials from the producing conv's epilogue
// (one per pixel tile and group, of the values as stored: no bias on read),
// so the stream is read once, by the apply pass.
void launch_groupnorm_partials(const float *x, int M, int cp, int c_real, int groups, const float *gamma,
                               const float *beta, int silu, float eps, const float *part, int nchunk, float *tab,
                               _Float16 *y, hipStream_t s)
{
    if (M <= 0) return;
    const int nt = stats_threads(cp);
    float *offset = tab, *scale = offset + cp, *shift = scale + cp;
    const int cpg = c_real / groups;
    hipLaunchKernelGGL(k_gn_final, dim3(groups), dim3(256), 0, s, part, nchunk, cp, c_real, cpg, eps,
                       static_cast<const float *>(nullptr), gamma, beta, offset, scale, shift);
    const int rl = nt / (cp / 4);
    const int64_t blocks = ((int64_t)M + (int64_t)rl * AU - 1) / ((int64_t)rl * AU);
    hipLaunchKernelGGL(k_gn_apply, dim3((unsigned)blocks), dim3(nt), 0, s, x, M, cp, offset, scale, shift, silu, y);
}

}  // namespace ig
