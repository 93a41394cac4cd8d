// The plain NT GEMM C[M][N] = oscale * A[M][K] . B[N][K]^T for gfx950: the
// decoder's 1x1 convs and the attention's products, with epilogues for
// f32 / f16 output (bias, residual add), and for the attention's softmax:
// per-row partial (max, sum of exp) statistics of the scaled scores, and
// the normalised probabilities from the rows' final statistics.
//
// Page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs": module doc (1x1
// convs as plain GEMMs, f16 inputs, f32 accumulation), `mmc` (B is the
// weight plane [N][K]) and `attention` (S = Q.K^T / sqrt(C) in f32, a row
// softmax to f16 P, O = P.V over query chunks). Page "cortiq-engine 0.7.6,
// src/vae.rs", `AttnBlock::apply`, for the max-subtracted softmax.
//
// Design:
//  * a workgroup of 8 wave64s owns a BM x BN tile; the waves form a WM x
//    (8 / WM) grid and each computes its (BM / WM) x (BN / (8 / WM)) block
//    as 32x32 tiles of v_mfma_f32_32x32x16_f16, with B as the MFMA's A
//    operand and A as its B operand: a lane's results are then runs of 4
//    consecutive columns of one row of C, stored 16 (f32) or 8 (f16) bytes
//    at a time straight from registers;
//  * K advances 64 per stage; stages are double-buffered in LDS and filled
//    by direct-to-LDS buffer loads (each lane's source offset fixed per
//    tile, the stage moving the scalar offset; rows past M read zero). Each
//    wave spreads its share of the next stage's loads over its four K steps;
//  * an LDS row holds 64 halves as 8 units of 16 bytes, unit u stored at
//    u ^ ((row >> 1) & 7): the fragment reads of 32 consecutive rows then
//    touch distinct bank groups in every pass;
//  * tiles run in groups of 8 M-tiles sweeping all N-tiles, dealt so each
//    XCD works on consecutive groups (the group's A rows and the B rows in
//    flight stay in its L2);
//  * softmax without a score matrix: a first pass writes, per row and per
//    64-column block, the block's max m_b and sum of exp(s - m_b) over the
//    valid columns; a reduction combines them into the row's (max, 1 / sum);
//    a second pass recomputes the same scores (same instruction sequence,
//    so the same values) and writes P = f16(exp(s - max) / sum), zero past
//    the valid columns.
#include <math.h>

#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NT = 512;   // 8 waves
constexpr int KST = 64;   // K per stage
constexpr int UPR = 8;    // 16-byte units per LDS row (KST halves)
constexpr int GROUP = 8;  // M-tiles per tile group
// a byte offset past every buffer read here (the launcher keeps buffers
// below it), with room for the stage offsets added to it
constexpr unsigned kOOB = 0xf0000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// merge partial softmax statistics (max, sum of exp(s - max))
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

template <int BM, int BN, int WM, int EPI>
__global__ __launch_bounds__(NT) void k_gemm2(Gemm2Args p)
{
    constexpr int WN = 8 / WM;
    constexpr int TM = BM / WM, TN = BN / WN;  // a wave's block
    constexpr int FM = TM / 32, FN = TN / 32;  // its MFMA tiles
    constexpr int A_INSTR = BM / 8, B_INSTR = BN / 8;  // a wave load fills 8 rows
    constexpr int T_INSTR = A_INSTR + B_INSTR;
    constexpr int PER_WAVE = T_INSTR / 8;
    constexpr int STAGE = (BM + BN) * UPR;
    static_assert(T_INSTR % 8 == 0 && FM >= 1 && FN >= 1, "tile shape");

    __shared__ __attribute__((aligned(16))) u32x4 lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // uniform (scalar branches); the mask tells the compiler wave < 8
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
    const int wm = wave / WN, wn = wave % WN;
    const int fx = lane & 31, fh = lane >> 5;

    const int M = p.M, N = p.N;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int per_group = GROUP * tiles_n;
    const int g = bid / per_group, first = g * GROUP;
    const int gsz = (tiles_m - first) < GROUP ? (tiles_m - first) : GROUP;
    const int local = bid - g * per_group;
    const int m0 = (first + local % gsz) * BM;
    int n0 = (local / gsz) * BN;
    // a pair of products: the tile's half of the columns picks its B, C, bias
    const bool second = p.nsplit > 0 && n0 >= p.nsplit;
    const _Float16 *bmat = second ? p.b2 : p.b;
    void *cmat = second ? p.c2 : p.c;
    const float *bvec = second ? p.bias2 : p.bias;
    const int nb = p.nsplit > 0 ? (second ? N - p.nsplit : p.nsplit) : N;  // B rows of this half
    if (second) n0 -= p.nsplit;

    const __amdgpu_buffer_rsrc_t a_src = make_rsrc(p.a, (uint32_t)((uint64_t)M * p.lda * 2));
    const __amdgpu_buffer_rsrc_t b_src = make_rsrc(bmat, (uint32_t)((uint64_t)nb * p.ldb * 2));

    // this lane's source offset for each of its wave's loads: load
    // ii = wave + 8k fills LDS units ii*64 .. ii*64+63, i.e. rows 8ii..8ii+7
    // of the A tile, then of the B tile; unit u of a row takes K units
    // u ^ ((row >> 1) & 7)
    unsigned voff[PER_WAVE];
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int ii = wave + 8 * k;
        const int r8 = lane >> 3, u = lane & 7;
        if (ii < A_INSTR) {
            const int row = 8 * ii + r8;
            const int ku = u ^ ((row >> 1) & 7);
            voff[k] = (m0 + row < M) ? ((unsigned)(m0 + row) * (unsigned)p.lda + 8u * ku) * 2u : kOOB;
        } else {
            const int row = 8 * (ii - A_INSTR) + r8;
            const int ku = u ^ ((row >> 1) & 7);
            voff[k] = ((unsigned)(n0 + row) * (unsigned)p.ldb + 8u * ku) * 2u;
        }
    }
    auto issue = [&](int st, int buf, int k0, int k1) __attribute__((always_inline)) {
        u32x4 *base = lds + buf * STAGE;
#pragma unroll
        for (int k = k0; k < k1; ++k) {
            const int ii = wave + 8 * k;
            if (ii < A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(a_src, (lds_void *)(base + ii * 64), 16, (int)voff[k],
                                                         st * KST * 2, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(b_src, (lds_void *)(base + ii * 64), 16, (int)voff[k],
                                                         st * KST * 2, 0, 0);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nst = p.K / KST;
    const int swz = (fx >> 1) & 7;  // rows wm*TM + 32i + fx share bits 1..3 with fx
    issue(0, 0, 0, PER_WAVE);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        const u32x4 *sA = lds + buf * STAGE;
        const u32x4 *sB = sA + BM * UPR;
        // each K step reads the next step's fragments before its MFMAs, so
        // the LDS latency hides behind them
        half8 af[2][FM], bf[2][FN];
        auto frags = [&](int ks, half8 *a, half8 *b) __attribute__((always_inline)) {
            const int unit = (2 * ks + fh) ^ swz;
#pragma unroll
            for (int i = 0; i < FM; ++i) a[i] = __builtin_bit_cast(half8, sA[(wm * TM + 32 * i + fx) * UPR + unit]);
#pragma unroll
            for (int j = 0; j < FN; ++j) b[j] = __builtin_bit_cast(half8, sB[(wn * TN + 32 * j + fx) * UPR + unit]);
        };
        frags(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < KST / 16; ++ks) {
            if (st + 1 < nst) issue(st + 1, buf ^ 1, ks * PER_WAVE / 4, (ks + 1) * PER_WAVE / 4);
            if (ks + 1 < KST / 16) frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[ks & 1][j], af[ks & 1][i], acc[i][j], 0, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // epilogue: accumulator (i, j) register 4q + e of this lane is C[m][n]
    // with m = m0 + wm*TM + 32i + fx, n = n0 + wn*TN + 32j + 8q + 4fh + e
    const float osc = p.oscale;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + 32 * i + fx;
        if (EPI == kEpiStats) {
            float mx = -INFINITY, sm = 0.f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = n0 + wn * TN + 32 * j + 8 * (r >> 2) + 4 * fh + (r & 3);
                    if (n < p.valid) mx = fmaxf(mx, osc * acc[i][j][r]);
                }
            if (mx != -INFINITY) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int n = n0 + wn * TN + 32 * j + 8 * (r >> 2) + 4 * fh + (r & 3);
                        if (n < p.valid) sm += __expf(osc * acc[i][j][r] - mx);
                    }
            }
            ms_merge(mx, sm, __shfl_xor(mx, 32), __shfl_xor(sm, 32));
            if (fh == 0 && m < M) {
                const int nparts = tiles_n * WN, part = (n0 / BN) * WN + wn;
                *reinterpret_cast<f32x2 *>(p.stats + 2 * ((int64_t)m * nparts + part)) = f32x2{mx, sm};
            }
            continue;
        }
        if (m >= M) continue;
        f32x2 rs = {0.f, 0.f};
        if (EPI == kEpiProb) rs = *reinterpret_cast<const f32x2 *>(p.rowstat + 2 * (int64_t)m);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * TN + 32 * j + 8 * q + 4 * fh;
                f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if (EPI == kEpiProb) {
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (n + e < p.valid) ? __expf(osc * v[e] - rs[0]) * rs[1] : 0.f;
                    half4v h = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
                    *reinterpret_cast<half4v *>(reinterpret_cast<_Float16 *>(cmat) + (int64_t)m * p.ldc + n) = h;
                    continue;
                }
                v *= osc;
                if (bvec) v += *reinterpret_cast<const f32x4 *>(bvec + n);
                if (EPI == kEpiF16) {
                    half4v h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                    *reinterpret_cast<half4v *>(reinterpret_cast<_Float16 *>(cmat) + (int64_t)m * p.ldc + n) = h;
                } else {
                    f32x4 *dst = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(cmat) + (int64_t)m * p.ldc + n);
                    if (p.accumulate) v += *dst;
                    *dst = v;
                }
            }
    }
}

// rowstat[r] = (max, 1 / sum) of row r from its nparts partial statistics;
// one wave per row
__global__ __launch_bounds__(256) void k_rowstat(const float *__restrict__ stats, int nparts, int rows,
                                                 float *__restrict__ rowstat)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    float m = -INFINITY, s = 0.f;
    for (int k = lane; k < nparts; k += 64) {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(stats + 2 * ((int64_t)row * nparts + k));
        ms_merge(m, s, v[0], v[1]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ms_merge(m, s, __shfl_xor(m, off), __shfl_xor(s, off));
    if (lane == 0) *reinterpret_cast<f32x2 *>(rowstat + 2 * (int64_t)row) = f32x2{m, 1.0f / s};
}

template <int BM, int BN, int WM, int EPI>
void launch_t(const Gemm2Args &a, hipStream_t s)
{
    const int grid = ((a.M + BM - 1) / BM) * (a.N / BN);
    hipLaunchKernelGGL((k_gemm2<BM, BN, WM, EPI>), dim3(grid), dim3(NT), 0, s, a);
}

template <int EPI>
void launch_e(const Gemm2Args &a, hipStream_t s)
{
    const int64_t tiles256 = ((int64_t)a.M + 255) / 256;
    if (a.N % 256 == 0) {
        if (tiles256 * (a.N / 256) >= 256) launch_t<256, 256, 2, EPI>(a, s);
        else launch_t<128, 256, 2, EPI>(a, s);
    } else if (a.N % 128 == 0) {
        launch_t<256, 128, 4, EPI>(a, s);
    } else {
        launch_t<256, 64, 4, EPI>(a, s);
    }
}

}  // namespace

bool gemm2_supported(const Gemm2Args &a)
{
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    if (a.M <= 0 || a.N <= 0 || a.K <= 0) return false;
    if (a.K % KST || a.N % 64 || a.lda % 8 || a.ldb % 8 || a.ldc % 4) return false;
    if (!al16(a.a) || !al16(a.b) || !al16(a.c) || (a.bias && !al16(a.bias))) return false;
    if ((uint64_t)a.M * a.lda * 2 >= kOOB) return false;
    if (a.nsplit > 0) {
        // two products: both halves tile by 256 columns, so no tile straddles
        const int n2 = a.N - a.nsplit;
        if (a.nsplit % 256 || n2 <= 0 || n2 % 256) return false;
        if (!al16(a.b2) || !al16(a.c2) || (a.bias2 && !al16(a.bias2))) return false;
        if (a.lda < a.K || a.ldb < a.K || a.ldc < (a.nsplit > n2 ? a.nsplit : n2)) return false;
        return (uint64_t)a.nsplit * a.ldb * 2 < kOOB && (uint64_t)n2 * a.ldb * 2 < kOOB;
    }
    if (a.lda < a.K || a.ldb < a.K || a.ldc < a.N) return false;
    // the buffer resources span M*lda and N*ldb halves; offsets stay below kOOB
    return (uint64_t)a.N * a.ldb * 2 < kOOB;
}

void launch_gemm2(int epi, const Gemm2Args &a, hipStream_t s)
{
    if (a.nsplit > 0 && epi != kEpiF32 && epi != kEpiF16) return;
    switch (epi) {
    case kEpiF32: launch_e<kEpiF32>(a, s); break;
    case kEpiF16: launch_e<kEpiF16>(a, s); break;
    case kEpiStats: launch_e<kEpiStats>(a, s); break;
    default: launch_e<kEpiProb>(a, s); break;
    }
}

int gemm2_stat_parts(int N)
{
    if (N % 256 == 0) return (N / 256) * 4;
    if (N % 128 == 0) return (N / 128) * 2;
    return (N / 64) * 2;
}

void launch_rowstat(const float *stats, int nparts, int rows, float *rowstat, hipStream_t s)
{
    if (rows <= 0) return;
    hipLaunchKernelGGL(k_rowstat, dim3((rows + 3) / 4), dim3(256), 0, s, stats, nparts, rows, rowstat);
}

}  // namespace ig
