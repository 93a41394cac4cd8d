// The decoder's last 3x3 convolution, whose output has only a few real
// channels (RGB), written straight into the NCHW frame with the bias:
// out[o][p] = b[o] + sum_{tap, c} W[o][tap][c] x[src(p, tap)][c], o < cout.
//
// Page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs", `output_rows`
// (conv_out on the normalised stream, then OUT_SRC: NHWC rows + bias into
// the NCHW frame); page "cortiq-engine 0.7.6, src/vae.rs", `Conv2d::apply`
// (stride 1, zero padding 1).
//
// Padding the output channels to the convolution kernels' 64 would make
// this the decoder's most expensive conv (21x the useful MFMA work, plus an
// f32 [M][64] intermediate and a transpose pass). Here the output channels
// are the 16 rows of a v_mfma_f32_16x16x32_f16 (weights as the A operand,
// channels >= cout zero) and 16 pixels its columns, so lanes 0..15 hold the
// real channels of 16 consecutive pixels and store them as 64-byte runs of
// NCHW rows. The convolution is then bound by reading its f16 input once.
//  * a workgroup of 4 waves owns 8 rows x 32 columns of output pixels; each
//    wave 2 rows, i.e. 4 groups of 16 pixels; three workgroups share a CU,
//    so enough loads are in flight to cover HBM latency;
//  * the reduction runs in stages of 32 input channels: the (8+2) x (32+2)
//    patch of the stage's channels streams into double-buffered LDS by
//    direct-to-LDS loads (zero outside the image); the stage's weights (9
//    taps, the lane's output channel, 8 of the 32 channels) are read from
//    the blocked weight plane into registers one stage ahead;
//  * a patch pixel's 32 channels are 4 units of 16 bytes, unit u stored at
//    u ^ ((pixel >> 2) & 3), so the 16 lanes reading one unit of 16
//    consecutive pixels touch 16 distinct bank groups;
//  * each XCD works on a contiguous band of tiles (workgroups are dealt to
//    the XCDs round robin), so neighbouring tiles' halo rows hit its L2;
//  * at most 3 output channels (the RGB frame) take a second form,
//    k_conv_out_taps: the nine taps' products side by side as the MFMA's
//    columns, summed from LDS afterwards.
#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NT = 256;                     // 4 waves
constexpr int OH = 8, OW = 32;              // output tile
constexpr int RPW = OH / 4;                 // output rows per wave
constexpr int PH = OH + 2, PW = OW + 2;     // input patch
constexpr int CS = 32;                      // input channels per stage
constexpr int UPP = CS * 2 / 16;            // 16-byte units per patch pixel
constexpr int A_UNITS = PH * PW * UPP;
constexpr int A_INSTR = (A_UNITS + 63) / 64;
constexpr int STAGE = A_INSTR * 64;         // units per stage buffer
constexpr int PER_WAVE = (A_INSTR + 3) / 4;
constexpr unsigned kOOB = 0xfffff000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__global__ __launch_bounds__(NT) void k_conv_out(const _Float16 *__restrict__ x, int H, int W, int cin_p,
                                                 const _Float16 *__restrict__ plane, int cout, int cout_p,
                                                 const float *__restrict__ bias, float *__restrict__ out,
                                                 int r0, int r1, int64_t HWo)
{
    __shared__ __attribute__((aligned(16))) u32x4 lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;  // pixel column in a group; K quarter / output row block

    // workgroups are dealt round robin to the 8 XCDs: remap so each XCD
    // takes a contiguous band of tiles, whose shared halo rows then come
    // from its own L2
    const int tiles_x = (W + OW - 1) / OW;
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int y0 = (bid / tiles_x) * OH, x0 = (bid % tiles_x) * OW;
    const __amdgpu_buffer_rsrc_t src = make_rsrc(x, (uint32_t)H * W * cin_p * 2);

    // this lane's source offset (stage 0) for each of its wave's patch loads
    unsigned aoff[PER_WAVE];
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int u = (wave + 4 * k) * 64 + lane;
        const int pix = u / UPP, su = u % UPP;
        const int cu = su ^ ((pix >> 2) & 3);  // stored unit -> channel unit
        const int pr = pix / PW, pc = pix % PW;
        const int sy = y0 - 1 + pr, sx = x0 - 1 + pc;
        const bool ok = (u < A_UNITS) & (sy >= 0) & (sy < H) & (sx >= 0) & (sx < W);
        aoff[k] = ok ? ((unsigned)(sy * W + sx) * (unsigned)cin_p + 8u * cu) * 2u : kOOB;
    }
    auto issue = [&](int st, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < PER_WAVE; ++k) {
            const int ii = wave + 4 * k;
            if (ii < A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void *)(lds + buf * STAGE + ii * 64), 16,
                                                         (int)aoff[k], st * CS * 2, 0, 0);
        }
    };

    constexpr int NG = RPW * OW / 16;  // groups of 16 pixels per wave
    f32x4 acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A operand: output channel o = lane % 16, channels 8 * (lane / 16) ..
    // + 7 of the stage; zero for o >= cout
    const int o = col;
    const int nst = cin_p / CS;
    // the stage's weights: blocked plane [cin_p/16][9][cout_p][16], channel
    // 32 st + 8 grp + e. They are read one stage ahead, before the next
    // stage's patch loads: loads complete in order, so a wait for weights
    // read after those would wait for the patch too
    auto load_w = [&](int st, half8 *wt) __attribute__((always_inline)) {
        const int c16 = 2 * st + (grp >> 1), ci = 8 * (grp & 1);
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            if (o < cout)
                wt[t] = *reinterpret_cast<const half8 *>(plane + ((int64_t)(c16 * 9 + t) * cout_p + o) * 16 + ci);
            else
                wt[t] = half8{};
        }
    };
    half8 wt[9], wn[9];
    load_w(0, wt);
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) {
            load_w(st + 1, wn);
            issue(st + 1, buf ^ 1);
        }
        const u32x4 *sA = lds + buf * STAGE;
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int dy = t / 3, dx = t % 3;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                // group g of this wave: output row RPW wave + g / (OW / 16), columns 16 (g % (OW / 16)) ..
                const int pr = RPW * wave + g / (OW / 16) + dy, pc = 16 * (g % (OW / 16)) + col + dx;
                const int pix = pr * PW + pc;
                const half8 xf = __builtin_bit_cast(half8, sA[pix * UPP + (grp ^ ((pix >> 2) & 3))]);
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wt[t], xf, acc[g], 0, 0, 0);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 9; ++t) wt[t] = wn[t];
    }
    // lane (grp, col) holds output channels 4 grp + r of pixel column col;
    // rows r0 .. r1 - 1 are stored, output planes HWo apart
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bv[r] = (bias && 4 * grp + r < cout) ? bias[4 * grp + r] : 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int oy = y0 + RPW * wave + g / (OW / 16), ox = x0 + 16 * (g % (OW / 16)) + col;
        if (oy < r0 || oy >= r1 || ox >= W) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ch = 4 * grp + r;
            if (ch < cout) out[ch * HWo + (int64_t)oy * W + ox] = acc[g][r] + bv[r];
        }
    }
}

// Output convs of at most 3 channels: the nine taps side by side. A
// v_mfma_f32_32x32x16_f16 takes 32 patch pixels as rows and the 27 (tap,
// output channel) pairs as columns, C[q][3 t + o] = sum_c x[q][c] w[o][c][t]
// over every pixel q of the tile's patch; then
// out[p][o] = b[o] + sum_t C[p + shift(t)][3 t + o] from LDS. Each input
// fragment is read from LDS once instead of once per tap, and the MFMA work
// per output pixel falls from 9 x 16 channel rows to (patch / tile) x 32
// columns, about a third. Same tile, patch stages and weight plane as the
// one-tap form above.
constexpr int TB = (PH * PW + 31) / 32;   // 32-pixel blocks of the patch
constexpr int NBW = (TB + 3) / 4;         // blocks per wave
constexpr int CP = 28;                    // LDS pitch (floats) of a patch pixel's 27 products
static_assert(TB * 32 * UPP <= STAGE, "the last block's padding rows stay inside the stage buffer");
static_assert(PH * PW * CP * 4 <= 2 * STAGE * 16, "the products fit the two stage buffers");

__global__ __launch_bounds__(NT) void k_conv_out_taps(const _Float16 *__restrict__ x, int H, int W, int cin_p,
                                                      const _Float16 *__restrict__ plane, int cout, int cout_p,
                                                      const float *__restrict__ bias, float *__restrict__ out,
                                                      int r0, int r1, int64_t HWo)
{
    __shared__ __attribute__((aligned(16))) u32x4 lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, h = lane >> 5;

    const int tiles_x = (W + OW - 1) / OW;
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    // tiles column by column within each XCD's range, so vertical
    // neighbours (which share the larger halo) run back to back: 3% faster
    // than row order at 1024^2 x 128
    const int tiles_y = (H + OH - 1) / OH;
    const int y0 = (bid % tiles_y) * OH, x0 = (bid / tiles_y) * OW;
    const __amdgpu_buffer_rsrc_t src = make_rsrc(x, (uint32_t)H * W * cin_p * 2);

    unsigned aoff[PER_WAVE];
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int u = (wave + 4 * k) * 64 + lane;
        const int pix = u / UPP, su = u % UPP;
        const int cu = su ^ ((pix >> 2) & 3);
        const int pr = pix / PW, pc = pix % PW;
        const int sy = y0 - 1 + pr, sx = x0 - 1 + pc;
        const bool ok = (u < A_UNITS) & (sy >= 0) & (sy < H) & (sx >= 0) & (sx < W);
        aoff[k] = ok ? ((unsigned)(sy * W + sx) * (unsigned)cin_p + 8u * cu) * 2u : kOOB;
    }
    auto issue = [&](int st, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < PER_WAVE; ++k) {
            const int ii = wave + 4 * k;
            if (ii < A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void *)(lds + buf * STAGE + ii * 64), 16,
                                                         (int)aoff[k], st * CS * 2, 0, 0);
        }
    };

    // B operand: column n = r (tap n / 3, output channel n % 3), channels
    // 16 ks + 8 h .. + 7 of the stage's K step ks; zero past 27 or cout
    const int tap = r / 3, oc = r % 3;
    const bool live = r < 27 && oc < cout;
    auto load_w = [&](int st, half8 (&wt)[CS / 16]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < CS / 16; ++ks) {
            const int c16 = (CS / 16) * st + ks;
            wt[ks] = live ? *reinterpret_cast<const half8 *>(plane + ((int64_t)(c16 * 9 + tap) * cout_p + oc) * 16 + 8 * h)
                          : half8{};
        }
    };

    f32x16 acc[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

    const int nst = cin_p / CS;
    half8 wt[CS / 16], wn[CS / 16];
    load_w(0, wt);
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) {
            load_w(st + 1, wn);
            issue(st + 1, buf ^ 1);
        }
        const u32x4 *sA = lds + buf * STAGE;
#pragma unroll
        for (int ks = 0; ks < CS / 16; ++ks) {
#pragma unroll
            for (int i = 0; i < NBW; ++i) {
                const int b = wave + 4 * i;
                if (b < TB) {
                    // A operand: patch pixel 32 b + r, the K step's units 2 ks + h (stored swizzled)
                    const int px = 32 * b + r;
                    const half8 xf = __builtin_bit_cast(half8, sA[px * UPP + ((2 * ks + h) ^ ((px >> 2) & 3))]);
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf, wt[ks], acc[i], 0, 0, 0);
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < CS / 16; ++ks) wt[ks] = wn[ks];
    }

    // the products to LDS (over the stage buffers, read by no one now):
    // lane (r, h) register j of block b holds C[32 b + 8 (j / 4) + 4 h + j % 4][r]
    float *const cl = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int b = wave + 4 * i;
        if (b < TB && r < 27) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int q = 32 * b + 8 * (j >> 2) + 4 * h + (j & 3);
                if (q < PH * PW) cl[q * CP + r] = acc[i][j];
            }
        }
    }
    __syncthreads();

    // one output pixel per thread: the nine taps' products of its
    // neighbours, in tap order, then the bias; rows r0 .. r1 - 1 are stored
    const int oy = tid / OW, ox = tid % OW;
    const int gy = y0 + oy, gx = x0 + ox;
    if (gy < r0 || gy >= r1 || gx >= W) return;
    float s[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 9; ++t) {
        const int q = (oy + t / 3) * PW + ox + t % 3;
#pragma unroll
        for (int o = 0; o < 3; ++o) s[o] += cl[q * CP + 3 * t + o];
    }
#pragma unroll
    for (int o = 0; o < 3; ++o)
        if (o < cout) out[o * HWo + (int64_t)gy * W + gx] = s[o] + (bias ? bias[o] : 0.f);
}

}  // namespace

void launch_conv_out(const _Float16 *x, int H, int W, int cin_p, const _Float16 *plane, int cout, int cout_p,
                     const float *bias, float *out, hipStream_t s, int r0, int r1, int64_t HWo)
{
    if (H <= 0 || W <= 0) return;
    if (r1 < 0) {
        r0 = 0;
        r1 = H;
        HWo = (int64_t)H * W;
    }
    const int grid = ((H + OH - 1) / OH) * ((W + OW - 1) / OW);
    if (cout <= 3)
        hipLaunchKernelGGL(k_conv_out_taps, dim3(grid), dim3(NT), 0, s, x, H, W, cin_p, plane, cout, cout_p, bias,
                           out, r0, r1, HWo);
    else
        hipLaunchKernelGGL(k_conv_out, dim3(grid), dim3(NT), 0, s, x, H, W, cin_p, plane, cout, cout_p, bias, out,
                           r0, r1, HWo);
}

}  // namespace ig
