// The 3x3 convolutions (plain and nearest-2x upsampled) as an implicit GEMM
// that reuses each input patch across all nine taps, for gfx950.
//
// Page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs", module doc: every
// 3x3 conv an implicit GEMM with the nearest-2x upsample folded into the
// A-tile gather, f16 inputs, f32 accumulation; `Rec::conv_s` for the
// output (raw f32 times oscale); `qconv` for the weight plane's (tap,
// channel) order. Page "cortiq-engine 0.7.6, src/vae.rs", `Conv2d::apply`
// and `upsample2x`, for the definition (stride 1, zero padding 1).
//
// Design (not the pages' 128x64 cooperative-matrix tiling):
//  * a workgroup owns an output tile of 8 rows x 32 columns x BN channels;
//    its 4 wave64s split it 2 (rows) x 2 (channels): each wave computes 4
//    output rows x 32 columns x BN/2 channels as 4 x BN/64 tiles of
//    v_mfma_f32_32x32x16_f16 (one output row = one 32-row MFMA operand);
//  * the reduction runs in stages of 16 input channels. A stage brings into
//    LDS the input patch the tile needs -- (8+2) x (32+2) pixels, or
//    (4+2) x (16+2) half-resolution pixels for the folded upsample -- and
//    the 16-channel slice of all nine taps' weights. All nine taps then read
//    the same patch at shifted offsets, so every input byte is fetched once
//    per tile instead of once per tap;
//  * for each tap column dx a wave loads the fragments of the patch rows it
//    needs once and uses them for the three tap rows dy (output row r at
//    tap row dy reads patch row r + dy; for the upsample, (r + dy + 1) / 2);
//  * LDS rows are 32 bytes (16 channels): consecutive lanes read
//    consecutive 32-byte rows, which the gfx950 LDS serves without bank
//    conflicts; the patch is zero outside the image (buffer loads past the
//    resource return zero), which is the convolution's zero padding;
//  * the next stage's global loads are issued before the current stage's
//    72 MFMAs per wave and land in registers; two workgroups per CU
//    (48 KB of LDS each) overlap one's LDS refill with the other's MFMAs;
//  * workgroups are dealt round robin to the 8 XCDs; the tile order is
//    remapped so each XCD works on a contiguous band of rows (shared halos
//    and weights stay in its L2).
#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
template <int N>
using uvec = unsigned __attribute__((ext_vector_type(N)));

constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr int TH = 8;    // output rows per tile
constexpr int TW = 32;   // output columns per tile
constexpr int CK = 16;   // input channels per stage
constexpr int FM = 4;    // output rows per wave
constexpr int kOOB = 0x7fffffff;

template <int MODE>
struct Geo {
    // patch extent (pixels) and the patch rows one wave reads
    static constexpr int PH = (MODE == kConv3x3) ? TH + 2 : TH / 2 + 2;
    static constexpr int PW = (MODE == kConv3x3) ? TW + 2 : TW / 2 + 2;
    static constexpr int AROWS = (MODE == kConv3x3) ? FM + 2 : FM / 2 + 2;
    // first patch row of wave row-group wm
    __device__ static constexpr int row0(int wm) { return (MODE == kConv3x3) ? FM * wm : (FM / 2) * wm; }
    // patch row (relative to row0) read by wave output row i at tap row dy
    __device__ static constexpr int arow(int i, int dy)
    {
        return (MODE == kConv3x3) ? i + dy : ((FM * 0 + i + dy + 1) >> 1);
    }
    // patch column read by tile column x at tap column dx
    __device__ static int pcol(int x, int dx) { return (MODE == kConv3x3) ? x + dx : ((x + dx + 1) >> 1); }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int MODE, int BN>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void k_conv_halo(IgemmArgs p)
{
    using G = Geo<MODE>;
    constexpr int PH = G::PH, PW = G::PW, AROWS = G::AROWS;
    constexpr int A_UNITS = PH * PW * 2;  // 16-byte units (pixel, channel half) per stage
    constexpr int B_UNITS = 9 * BN * 2;   // (tap, n, channel half)
    constexpr int A_PER = (A_UNITS + NT - 1) / NT;
    constexpr int B_PER = (B_UNITS + NT - 1) / NT;
    constexpr int FN = BN / 64;  // 32-channel fragments per wave
    static_assert(A_PER <= 4, "patch units per thread");
    // the output tile leaves through LDS, two tile rows at a time
    constexpr int OUT_ROWS = 2;
    constexpr int OUT_BYTES = OUT_ROWS * TW * BN * 4;
    constexpr int STAGE_BYTES = (A_UNITS + B_UNITS) * 16;
    static_assert(OUT_BYTES <= STAGE_BYTES, "output staging fits the stage buffer");

    __shared__ __attribute__((aligned(16))) u32x4 lds[A_UNITS + B_UNITS];
    u32x4 *sA = lds;            // [PH * PW][2]
    u32x4 *sB = lds + A_UNITS;  // [9][BN][2]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int fx = lane & 31;  // tile column (A) / channel within a fragment (B)
    const int fh = lane >> 5;  // channel half of the stage: 8*fh .. 8*fh+7

    const int H = p.H, W = p.W, cin_p = p.cin_p, cout_p = p.N;
    const int Hout = (MODE == kConv3x3Up2) ? 2 * H : H;
    const int Wout = (MODE == kConv3x3Up2) ? 2 * W : W;
    const int tiles_x = (Wout + TW - 1) / TW;
    const int n_tiles = cout_p / BN;

    // XCD-aware tile order (channel tiles fastest, then columns, then rows)
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int ntile = bid % n_tiles;
    const int t2 = bid / n_tiles;
    const int y0 = (t2 / tiles_x) * TH, x0 = (t2 % tiles_x) * TW, n0 = ntile * BN;
    const int py0 = (MODE == kConv3x3) ? y0 - 1 : y0 / 2 - 1;
    const int px0 = (MODE == kConv3x3) ? x0 - 1 : x0 / 2 - 1;

    const __amdgpu_buffer_rsrc_t a_src = make_rsrc(p.a, (uint32_t)H * W * cin_p * 2);
    // stage st of the blocked plane [cin_p/16][9][cout_p][16]
    const int64_t b_stage = (int64_t)9 * cout_p * CK;
    const _Float16 *b_tile = p.b + (int64_t)n0 * CK;

    // byte offset (stage 0) of each patch unit this thread loads; kOOB for
    // pixels outside the image and for units past the patch
    int4v aoff = {kOOB, kOOB, kOOB, kOOB};
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int u = tid + NT * i;
        const int pix = u >> 1, half = u & 1;
        const int pr = pix / PW, pc = pix - (pix / PW) * PW;
        const int sy = py0 + pr, sx = px0 + pc;
        const bool ok = (u < A_UNITS) & (sy >= 0) & (sy < H) & (sx >= 0) & (sx < W);
        aoff[i] = ok ? ((sy * W + sx) * cin_p + half * 8) * 2 : kOOB;
    }

    uvec<4 * A_PER> ra;
    uvec<4 * B_PER> rb;
    auto gload = [&](int st) __attribute__((always_inline)) {
        const int cb = st * CK * 2;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int off = aoff[i] == kOOB ? kOOB : aoff[i] + cb;
            const u32x4 v = buf_load16(a_src, off);
            ra[4 * i + 0] = v.x;
            ra[4 * i + 1] = v.y;
            ra[4 * i + 2] = v.z;
            ra[4 * i + 3] = v.w;
        }
        const _Float16 *bs = b_tile + st * b_stage;
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int u = tid + NT * i;
            const int tap = u / (2 * BN);
            const int rem = u - tap * (2 * BN);  // n * 2 + half: contiguous within a tap
            u32x4 v = {0, 0, 0, 0};
            if (B_UNITS % NT == 0 || u < B_UNITS)
                v = *reinterpret_cast<const u32x4 *>(bs + (int64_t)tap * cout_p * CK + rem * 8);
            rb[4 * i + 0] = v.x;
            rb[4 * i + 1] = v.y;
            rb[4 * i + 2] = v.z;
            rb[4 * i + 3] = v.w;
        }
    };
    auto lstore = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int u = tid + NT * i;
            if (A_UNITS % NT == 0 || u < A_UNITS)
                sA[u] = u32x4{ra[4 * i], ra[4 * i + 1], ra[4 * i + 2], ra[4 * i + 3]};
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int u = tid + NT * i;
            if (B_UNITS % NT == 0 || u < B_UNITS)
                sB[u] = u32x4{rb[4 * i], rb[4 * i + 1], rb[4 * i + 2], rb[4 * i + 3]};
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ar0 = G::row0(wm);
    const int nst = cin_p / CK;

    gload(0);
    lstore();
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
        const bool more = st + 1 < nst;
        if (more) gload(st + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dx = 0; dx < 3; ++dx) {
            half8 af[AROWS];
            const int pc = G::pcol(fx, dx);
#pragma unroll
            for (int a = 0; a < AROWS; ++a)
                af[a] = __builtin_bit_cast(half8, sA[((ar0 + a) * PW + pc) * 2 + fh]);
#pragma unroll
            for (int dy = 0; dy < 3; ++dy) {
                const int tap = dy * 3 + dx;
                half8 bf[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bf[j] = __builtin_bit_cast(half8, sB[(tap * BN + wn * (BN / 2) + j * 32 + fx) * 2 + fh]);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[G::arow(i, dy)], bf[j],
                                                                           acc[i][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // every wave is done reading this stage
        if (more) {
            lstore();
            __syncthreads();
        }
    }

    // epilogue through LDS: accumulator element (i, j, r) of lane l is tile
    // pixel (4 wm + i, 8 (r / 4) + 4 (l / 32) + r % 4), channel
    // wn BN/2 + 32 j + l % 32. Pass q stages tile rows {q, q + 4} (wave row
    // i = q of both wave row groups) as [2][TW][BN] f32, then every thread
    // writes 16 contiguous bytes: each tile row leaves as one TW*BN*4-byte
    // run (contiguous in y when BN equals the output row width).
    const float osc = p.oscale;
    const bool accum = p.accumulate != 0;
    float *stg = reinterpret_cast<float *>(lds);
    float bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = p.bias ? p.bias[n0 + wn * (BN / 2) + j * 32 + fx] : 0.f;
    float *out = reinterpret_cast<float *>(p.c);
#pragma unroll
    for (int q = 0; q < FM; ++q) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int px = (r >> 2) * 8 + fh * 4 + (r & 3);
                stg[(wm * TW + px) * BN + wn * (BN / 2) + j * 32 + fx] = osc * acc[q][j][r] + bv[j];
            }
        __syncthreads();
        constexpr int V4 = OUT_ROWS * TW * BN / 4;  // 16-byte pieces in the staging area
#pragma unroll
        for (int v = tid; v < V4; v += NT) {
            const int e = v * 4;
            const int rr = e / (TW * BN);  // 0: tile row q, 1: tile row q + 4
            const int px = (e / BN) % TW;
            const int ch = e % BN;
            const int oy = y0 + rr * FM + q, ox = x0 + px;
            if (oy < Hout && ox < Wout) {
                float4 val = reinterpret_cast<const float4 *>(stg)[v];
                float *dst = out + ((int64_t)oy * Wout + ox) * p.ldc + n0 + ch;
                if (accum) {
                    const float4 o = *reinterpret_cast<const float4 *>(dst);
                    val.x += o.x;
                    val.y += o.y;
                    val.z += o.z;
                    val.w += o.w;
                }
                *reinterpret_cast<float4 *>(dst) = val;
            }
        }
        __syncthreads();
    }
}

template <int MODE, int BN>
void launch_t(const IgemmArgs &a, hipStream_t s)
{
    const int Hout = (MODE == kConv3x3Up2) ? 2 * a.H : a.H;
    const int Wout = (MODE == kConv3x3Up2) ? 2 * a.W : a.W;
    const int grid = ((Hout + TH - 1) / TH) * ((Wout + TW - 1) / TW) * (a.N / BN);
    hipLaunchKernelGGL((k_conv_halo<MODE, BN>), dim3(grid), dim3(NT), 0, s, a);
}

}  // namespace

void launch_conv_halo(int mode, const IgemmArgs &a, hipStream_t s)
{
    if (a.M <= 0) return;
    const bool bn128 = (a.N % 128) == 0;
    if (mode == kConv3x3) {
        if (bn128) launch_t<kConv3x3, 128>(a, s);
        else launch_t<kConv3x3, 64>(a, s);
    } else {
        if (bn128) launch_t<kConv3x3Up2, 128>(a, s);
        else launch_t<kConv3x3Up2, 64>(a, s);
    }
}

}  // namespace ig
