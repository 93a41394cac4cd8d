// The plain NT GEMM fallback for gfx950 and the dispatch of the decoder's
// products: C[M][N] = oscale * A.B^T (+ bias), the 1x1 convs and the
// attention's products (page "cortiq-engine 0.8.3,
// src/gpu_wgpu/qi21_vae.rs": module doc, 1x1 convs as plain GEMMs, f16
// inputs, f32 accumulation; `mmc`, B is the weight "plane" [N][K], A the
// activations). Shapes the direct-to-LDS GEMM (gemm2.hip) takes go there;
// the 3x3 convolutions go to their own kernels (conv_ws.hip, conv_halo.hip).
//
// This kernel takes the rest (K a multiple of 32, any M):
//  * one workgroup = 4 wave64s in a 2x2 grid, tile BM x BN (256|128 x
//    128|64); each wave owns a (BM/2) x (BN/2) block of 32x32 MFMA tiles,
//    v_mfma_f32_32x32x16_f16 with the f32 accumulators kept in registers;
//  * K advances 32 per step, global -> registers -> LDS, double-buffered,
//    the next step's loads in flight during the current step's MFMAs; one
//    barrier per step. LDS rows are 64 B of data + 16 B of padding so the
//    16-byte fragment reads of consecutive rows fall in different banks;
//  * rows past M read zero through the buffer resource's bound;
//  * the tile order is XCD-aware: workgroups are dealt round robin to the 8
//    XCDs, so block b is remapped to run tile (b % 8) * (grid / 8) + b / 8;
//  * the epilogue applies oscale, the bias and optionally the residual add
//    (y += ...) and writes f32 or f16 with rows >= M masked.
#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));  // per-thread row state, in registers
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte load

constexpr int BK = 32;           // K elements per pipeline step
constexpr int LDS_ROW = BK + 8;  // halves per LDS row (64 B data + 16 B pad)
constexpr int NT = 256;          // threads per workgroup

// Buffer resource over `bytes` bytes at `base`: loads at offsets at or past
// `bytes` return zero, which is how the gather reads the convolution's zero
// padding and masks rows past M without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}


__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int A_PER, int B_PER>
__device__ __forceinline__ void load_step(const IgemmArgs &p, __amdgpu_buffer_rsrc_t ra_src, int4v g_row,
                                          const _Float16 *b_base, int64_t b_stride, int q, int ks,
                                          u32x4 (&ra)[A_PER], u32x4 (&rb)[B_PER])
{
    const int kb = ks * BK;
#pragma unroll
    for (int j = 0; j < A_PER; ++j)  // rows past M are past the resource
        ra[j] = buf_load16(ra_src, (g_row[j] * p.lda + kb + q * 8) * 2);
#pragma unroll
    for (int j = 0; j < B_PER; ++j) rb[j] = *reinterpret_cast<const u32x4 *>(b_base + j * b_stride + kb);
}

template <int BM, int BN, int A_PER, int B_PER>
__device__ __forceinline__ void store_step(_Float16 (*sA)[LDS_ROW], _Float16 (*sB)[LDS_ROW], int rbase,
                                           int q, const u32x4 (&ra)[A_PER], const u32x4 (&rb)[B_PER])
{
#pragma unroll
    for (int j = 0; j < A_PER; ++j) *reinterpret_cast<u32x4 *>(&sA[rbase + 64 * j][q * 8]) = ra[j];
#pragma unroll
    for (int j = 0; j < B_PER; ++j) *reinterpret_cast<u32x4 *>(&sB[rbase + 64 * j][q * 8]) = rb[j];
}

template <int FM, int FN, int WTM, int WTN>
__device__ __forceinline__ void mma_step(const _Float16 (*sA)[LDS_ROW], const _Float16 (*sB)[LDS_ROW],
                                         int wm, int wn, int frow, int fk, f32x16 (&acc)[FM][FN])
{
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        half8 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *reinterpret_cast<const half8 *>(&sA[wm * WTM + i * 32 + frow][kk * 16 + fk]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = *reinterpret_cast<const half8 *>(&sB[wn * WTN + j * 32 + frow][kk * 16 + fk]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
}

template <int BM, int BN, bool OUT_F16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void k_igemm(IgemmArgs p)
{
    constexpr int WTM = BM / 2, WTN = BN / 2;        // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;      // 32x32 MFMA tiles per wave
    constexpr int A_PER = BM / 64, B_PER = BN / 64;  // 16-byte loads per thread per step
    static_assert(A_PER <= 4, "row state holds at most 4 rows");

    __shared__ __attribute__((aligned(16))) _Float16 sA[2][BM][LDS_ROW];
    __shared__ __attribute__((aligned(16))) _Float16 sB[2][BN][LDS_ROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware tile order
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int n_tiles = p.N / BN;
    const int mt = bid / n_tiles, ntile = bid - mt * n_tiles;
    const int m0 = mt * BM, n0 = ntile * BN;

    const int q = tid & 3;       // which 16-byte chunk of the 64-byte K slice
    const int rbase = tid >> 2;  // 0..63: row within each group of 64

    // the block's rows only: offsets stay small, rows past M read zero
    const int rows = (p.M - m0) < BM ? (p.M - m0) : BM;
    const __amdgpu_buffer_rsrc_t a_src = make_rsrc(p.a + (int64_t)m0 * p.lda, (uint32_t)rows * p.lda * 2);
    int4v g_row = {0, 0, 0, 0};  // the block rows this thread loads
#pragma unroll
    for (int j = 0; j < A_PER; ++j) g_row[j] = rbase + 64 * j;
    // B rows n0 + rbase + 64j
    const _Float16 *b_base = p.b + (int64_t)(n0 + rbase) * p.ldb + q * 8;
    const int64_t b_stride = (int64_t)64 * p.ldb;

    const int nks = p.K / BK;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int frow = lane & 31;      // fragment row (A) / column (B)
    const int fk = (lane >> 5) * 8;  // this lane's 8 K elements within 16

    u32x4 ra[A_PER], rb[B_PER];
    load_step<A_PER, B_PER>(p, a_src, g_row, b_base, b_stride, q, 0, ra, rb);
    store_step<BM, BN, A_PER, B_PER>(sA[0], sB[0], rbase, q, ra, rb);
    __syncthreads();

    int cur = 0;
    for (int ks = 0; ks < nks - 1; ++ks) {
        // the next step's loads go out first and stay first: the MFMAs of
        // this step hide their latency
        load_step<A_PER, B_PER>(p, a_src, g_row, b_base, b_stride, q, ks + 1, ra, rb);
        __builtin_amdgcn_sched_barrier(0);
        mma_step<FM, FN, WTM, WTN>(sA[cur], sB[cur], wm, wn, frow, fk, acc);
        __builtin_amdgcn_sched_barrier(0);
        store_step<BM, BN, A_PER, B_PER>(sA[cur ^ 1], sB[cur ^ 1], rbase, q, ra, rb);
        __syncthreads();
        cur ^= 1;
    }
    mma_step<FM, FN, WTM, WTN>(sA[cur], sB[cur], wm, wn, frow, fk, acc);

    // epilogue: lane holds column (lane & 31) of each 32x32 tile, rows
    // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r
    const float osc = p.oscale;
    const bool accum = p.accumulate != 0;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WTN + j * 32 + frow;
        const float bv = p.bias ? p.bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row < p.M) {
                    float v = osc * acc[i][j][r] + bv;
                    const int64_t off = (int64_t)row * p.ldc + col;
                    if (OUT_F16) {
                        reinterpret_cast<_Float16 *>(p.c)[off] = (_Float16)v;
                    } else {
                        float *cp = reinterpret_cast<float *>(p.c) + off;
                        if (accum) v += *cp;
                        *cp = v;
                    }
                }
            }
        }
    }
}

template <int BM, int BN, bool F16>
void launch_t(const IgemmArgs &a, hipStream_t s)
{
    const int mt = (a.M + BM - 1) / BM;
    const int grid = mt * (a.N / BN);
    hipLaunchKernelGGL((k_igemm<BM, BN, F16>), dim3(grid), dim3(NT), 0, s, a);
}

template <bool F16>
void launch_mode(const IgemmArgs &a, hipStream_t s)
{
    const bool bn128 = (a.N % 128) == 0;
    const int bn = bn128 ? 128 : 64;
    // prefer the 256-row tile when it still gives two workgroups per CU
    const long tiles256 = (long)((a.M + 255) / 256) * (a.N / bn);
    const bool bm256 = tiles256 >= 512;
    if (bm256 && bn128) launch_t<256, 128, F16>(a, s);
    else if (bm256) launch_t<256, 64, F16>(a, s);
    else if (bn128) launch_t<128, 128, F16>(a, s);
    else launch_t<128, 64, F16>(a, s);
}

}  // namespace

void launch_igemm(int mode, const IgemmArgs &a, hipStream_t s)
{
    if (a.M <= 0) return;
    switch (mode) {
    case kGemm: {
        // the direct-to-LDS GEMM when the shapes allow it
        Gemm2Args g{};
        g.a = a.a;
        g.b = a.b;
        g.c = a.c;
        g.bias = a.bias;
        g.M = a.M;
        g.N = a.N;
        g.K = a.K;
        g.lda = a.lda;
        g.ldb = a.ldb;
        g.ldc = a.ldc;
        g.accumulate = a.accumulate;
        g.oscale = a.oscale;
        if (gemm2_supported(g) && !(a.out_f16 && a.accumulate)) {
            launch_gemm2(a.out_f16 ? kEpiF16 : kEpiF32, g, s);
        } else if (a.out_f16) {
            launch_mode<true>(a, s);
        } else {
            launch_mode<false>(a, s);
        }
        break;
    }
    case kConv3x3:
    case kConv3x3Up2: launch_conv_halo(mode, a, s); break;
    default: break;
    }
}

}  // namespace ig
