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
//  * a workgroup owns an output tile of 16 rows x 32 columns x BN
//    channels: 4 wave64s with BN = 64 (two workgroups per CU, so one's
//    epilogue overlaps the other's MFMAs), each wave 4 output rows x 32
//    columns x 64 channels; for a plain conv with no more tiles than CUs, 8
//    waves with BN = 64 (4 rows x 32 channels each, two waves per SIMD);
//    8 waves with BN = 128 when the fused RMS_norm needs all 128 channels
//    of a pixel in one tile. A wave's block is 4 x FN tiles of
//    v_mfma_f32_32x32x16_f16 (one output row is one 32-row MFMA operand);
//  * the reduction runs in stages of 16 input channels. A stage brings into
//    LDS the input patch the tile needs -- (16+2) x (32+2) pixels, or
//    (8+2) x (16+2) half-resolution pixels for the folded upsample -- and
//    the 16-channel slice of all nine taps' weights (one contiguous block
//    of the [cin_p/16][9][cout_p][16] plane). All nine taps read the same
//    patch at shifted offsets, so every input byte is fetched once per tile;
//  * stages are double-buffered in LDS and filled by direct-to-LDS buffer
//    loads (buffer_load ... lds): the next stage streams in while the
//    current one feeds 72 MFMAs per wave, with no register staging and one
//    barrier per stage. A wave issues its share of the next stage's loads a
//    few at a time between its first seven MFMA groups (patch loads first),
//    so no wave waits on a burst of load issues before its first MFMA and
//    the last loads have two groups' time to land. Loads past the image
//    return zero, which is the convolution's zero padding;
//  * for each tap column dx a wave loads the fragments of the patch rows it
//    needs once and uses them for the three tap rows dy (output row r at
//    tap row dy reads patch row r + dy; for the upsample, (r + dy + 1) / 2).
//    Each tap group reads the next group's weight fragments (and, at the
//    last dy, the next column's patch fragments) before its own MFMAs, so
//    the LDS latency hides behind them;
//  * LDS holds a pixel's (or an output channel's) 16 channels as two
//    16-byte halves, the halves swapped on every other group of 8
//    columns: a fragment read (32 lanes on consecutive columns, the other
//    32 on the other half) then touches 16 distinct bank groups in each
//    pass, where the plain 32-byte pitch would conflict two ways;
//  * the f32 tile leaves through LDS: every tile row goes out as one
//    contiguous run of 16-byte stores; a conv that adds into the stream
//    (a template instantiation of its own) loads a pass's stream values
//    all together under the staging barrier;
//  * when the tile spans all of a pixel's channels (N = 64 or 128) the
//    epilogue can instead emit the pixel's RMS_norm (+ SiLU) as f16 from the
//    staged rows -- the next step of the pages' resnet and output recipes --
//    so the f32 result is neither stored nor read back;
//  * for a GroupNorm that follows, the epilogue can also gather the group
//    statistics of what it stores (per tile and group: count, mean and
//    sum of squared deviations), so the norm reads its input once
//    (page "cortiq-engine 0.8.72, src/gpu_wgpu/s2v_vae.rs", GN_PART_SRC,
//    whose per-workgroup partials come from a pass of their own);
//  * workgroups are dealt round robin to the 8 XCDs; the tile order is
//    remapped so each XCD works on a contiguous band of rows (shared halos
//    and weights stay in its L2).
#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int TH = 16;   // output rows per tile
constexpr int TW = 32;   // output columns per tile
constexpr int CK = 16;   // input channels per stage
constexpr int FM = 4;    // output rows per wave
constexpr int DG = 7;    // tap groups that issue the next stage's loads
// patch offset of pixels outside the image: past every input (inputs stay
// below kConvInMaxBytes), also after the stages' channel offsets are added
constexpr int kOOB = (int)kConvInMaxBytes;

template <int MODE>
struct Geo {
    // patch extent (pixels) and the patch rows one wave reads
    static constexpr int PH = (MODE == kConv3x3) ? TH + 2 : TH / 2 + 2;
    static constexpr int PW = (MODE == kConv3x3) ? TW + 2 : TW / 2 + 2;
    static constexpr int AROWS = (MODE == kConv3x3) ? FM + 2 : FM / 2 + 2;
    // first patch row of wave row group wm
    __device__ static constexpr int row0(int wm) { return (MODE == kConv3x3) ? FM * wm : (FM / 2) * wm; }
    // patch row (relative to row0) read by the wave's output row i at tap row dy
    __device__ static constexpr int arow(int i, int dy) { return (MODE == kConv3x3) ? i + dy : (i + dy + 1) >> 1; }
    // patch column read by tile column x at tap column dx
    __device__ static int pcol(int x, int dx) { return (MODE == kConv3x3) ? x + dx : ((x + dx + 1) >> 1); }
};

// Stage buffer size (16-byte units): the patch, padded to whole wave loads,
// then the nine taps' weights. A workgroup may walk several tiles only when
// its f32 output staging (RS rows x TW pixels per pass, a pixel's BN
// channels at a pitch of SP floats) fits one stage buffer, the one the next
// tile's first stage is not landing in.
template <int MODE, int BN>
constexpr int stage_units()
{
    return (Geo<MODE>::PH * Geo<MODE>::PW * 2 + 63) / 64 * 64 + 9 * BN * 2;
}
// Staging pitch: the 128-channel fused norm (8 lanes per pixel, 16
// channels each) keeps 8 floats of padding per staged pixel, chosen when its
// lanes read 32 channels each (4 lanes per pixel, 8 lanes then met on one
// bank group without it). The plain epilogue reads the rows linearly and
// needs none; the 64-channel norm (2 lanes per pixel, 32 channels each)
// keeps the plain pitch (padding it costs that instantiation spills).
template <int BN, bool NORM>
constexpr int stage_pitch()
{
    return (NORM && BN == 128) ? BN + 8 : BN;
}
// Tile rows staged per epilogue pass: 4 (one per wave row group), or 2 for
// the 128-channel fused norm, whose 4-row staging would not fit one stage
// buffer and so could not walk tiles
template <int BN, bool NORM>
constexpr int stage_rows()
{
    return (NORM && BN == 128) ? 2 : 4;
}
template <int MODE, int BN, bool NORM>
constexpr bool can_walk()
{
    return stage_rows<BN, NORM>() * TW * stage_pitch<BN, NORM>() * 4 <= stage_units<MODE, BN>() * 16;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// A tile: its origin, and a lane's sources for the tile's stage loads: the
// weight offset, and the patch offset (stage 0, bytes) of each patch load of
// its wave (load index ii = wave + NW k covers units ii*64 .. ii*64+63).
// (At namespace scope: a class local to the kernel template keeps hipcc's
// host pass from emitting the kernel's launch stub.)
struct Tile {
    int y0, x0, n0, b_lane;
    int8v aoff;
};

// GroupNorm statistics in the epilogue: (n, mean, M2) of a thread's values
// of one group, the batch of four channels of one pixel folded in by Chan,
// Golub and LeVeque's update (the batch's own mean and squared deviations
// first, so a large common offset does not cancel), and the merge of two
// such figures (across lanes and waves)
struct GnAcc {
    float n = 0.f, m = 0.f, q = 0.f;
    __device__ __forceinline__ void fold4(float4 v)
    {
        const float bm = 0.25f * ((v.x + v.y) + (v.z + v.w));
        const float d0 = v.x - bm, d1 = v.y - bm, d2 = v.z - bm, d3 = v.w - bm;
        const float bq = d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
        const float nn = n + 4.f, w = 4.f * __builtin_amdgcn_rcpf(nn), d = bm - m;
        m += d * w;
        q += bq + d * d * n * w;
        n = nn;
    }
    __device__ __forceinline__ void merge(float nb, float mb, float qb)
    {
        const float nn = n + nb;
        if (nb > 0.f) {
            const float w = nb / nn, d = mb - m;
            m += d * w;
            q += qb + d * d * n * w;
            n = nn;
        }
    }
};

template <int MODE, int BN, int NW, bool NORM, bool GNS = false, bool ACC = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(8 / NW)))
void k_conv_halo(IgemmArgs p)
{
    using G = Geo<MODE>;
    constexpr int NT = 64 * NW;                          // threads per workgroup
    constexpr int WN = NW / 4;                           // wave groups along the channels
    constexpr int PH = G::PH, PW = G::PW, AROWS = G::AROWS;
    constexpr int A_UNITS = PH * PW * 2;                 // 16-byte units (pixel, channel half)
    constexpr int A_INSTR = (A_UNITS + 63) / 64;         // wave loads per stage for the patch
    constexpr int A_PAD = A_INSTR * 64;                  // patch region, padded to whole loads
    constexpr int B_UNITS = 9 * BN * 2;                  // (tap, n, channel half)
    constexpr int B_INSTR = B_UNITS / 64;
    constexpr int T_INSTR = A_INSTR + B_INSTR;
    constexpr int PER_WAVE = (T_INSTR + NW - 1) / NW;
    constexpr int A_PER_WAVE = (A_INSTR + NW - 1) / NW;  // patch loads of the busiest wave
    constexpr int STAGE = A_PAD + B_UNITS;               // units per stage buffer
    static_assert(STAGE == stage_units<MODE, BN>(), "stage layout");
    constexpr int FN = BN / (32 * WN);                   // 32-channel fragments per wave
    static_assert(B_UNITS % 64 == 0, "whole weight loads");
    static_assert(A_PER_WAVE <= 8, "patch offsets per lane");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    // the output tile leaves through LDS, 4 tile rows per pass
    constexpr int SP = stage_pitch<BN, NORM>();
    constexpr int RS = stage_rows<BN, NORM>();  // rows staged per pass
    static_assert(RS * TW * SP * 4 <= 2 * STAGE * 16, "output staging fits the stage buffers");

    __shared__ __attribute__((aligned(16))) u32x4 lds[2 * STAGE];
    // the fused norm's gamma, read from LDS in the epilogue (a tile spans
    // all N = BN channels, so n0 = 0)
    __shared__ __attribute__((aligned(16))) float gam[NORM ? BN : 4];
    // the waves' GroupNorm partials of a tile: [wave][group of the tile][3]
    __shared__ float gns[GNS ? NW * 16 * 3 : 1];
    static_assert(!(GNS && (NORM || BN != 64)), "statistics from the plain 64-channel tiles");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // uniform (scalar branches); the mask tells the compiler wave < NW
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
    const int wm = wave / WN, wn = wave % WN;
    const int fx = lane & 31;  // tile column (A) / channel within a fragment (B)
    const int fh = lane >> 5;  // channel half of the stage: 8*fh .. 8*fh+7

    const int H = p.H, W = p.W, cin_p = p.cin_p, cout_p = p.N;
    const int Hout = (MODE == kConv3x3Up2) ? 2 * H : H;
    const int Wout = (MODE == kConv3x3Up2) ? 2 * W : W;
    const int tiles_x = (Wout + TW - 1) / TW;
    const int n_tiles = cout_p / BN;

    // Tile schedule (channel tiles fastest, then columns, then rows). With a
    // grid that is a multiple of 8, XCD x (workgroups bid = x mod 8) takes
    // the contiguous tile range [x T / 8, (x + 1) T / 8), so neighbouring
    // tiles share halos and weights in its L2; its j-th workgroup walks
    // tiles base + j, base + j + G / 8, ... (one tile when G = T).
    const int T = ((Hout + TH - 1) / TH) * tiles_x * n_tiles;
    const int nblk = gridDim.x;
    int t, t_end, t_step;
    if ((nblk & 7) == 0) {
        const int xcd = blockIdx.x & 7;
        t = (int)((int64_t)xcd * T / 8) + (blockIdx.x >> 3);
        t_end = (int)((int64_t)(xcd + 1) * T / 8);
        t_step = nblk >> 3;
    } else {
        t = blockIdx.x;
        t_end = T;
        t_step = nblk;
    }
    if (t >= t_end) return;  // uniform: the whole workgroup leaves

    const __amdgpu_buffer_rsrc_t a_src = make_rsrc(p.a, (uint32_t)H * W * cin_p * 2);
    // stage st of the blocked plane [cin_p/16][9][cout_p][16]
    const int b_stage = 9 * cout_p * CK;
    // weight unit (n, stored half) holds channel half stored ^ bit 3 of n.
    // Both operands load through buffer resources (MUBUF): a FLAT-encoded
    // LDS load would make the compiler drain every LDS read before each
    // MFMA group.
    const __amdgpu_buffer_rsrc_t b_src = make_rsrc(p.b, (uint32_t)(9 * cin_p) * cout_p * 2);
    const int b_half = (lane ^ ((lane >> 4) & 1)) * 8 * 2;

    auto make_tile = [&](int tt) __attribute__((always_inline)) {
        Tile r;
        const int ntile = tt % n_tiles;
        const int t2 = tt / n_tiles;
        r.y0 = (t2 / tiles_x) * TH;
        r.x0 = (t2 % tiles_x) * TW;
        r.n0 = ntile * BN;
        r.b_lane = r.n0 * CK * 2 + b_half;
        const int py0 = (MODE == kConv3x3) ? r.y0 - 1 : r.y0 / 2 - 1;
        const int px0 = (MODE == kConv3x3) ? r.x0 - 1 : r.x0 / 2 - 1;
        r.aoff = int8v{kOOB, kOOB, kOOB, kOOB, kOOB, kOOB, kOOB, kOOB};
#pragma unroll
        for (int k = 0; k < A_PER_WAVE; ++k) {
            const int u = (wave + NW * k) * 64 + lane;
            const int pix = u >> 1;
            const int pr = pix / PW, pc = pix - (pix / PW) * PW;
            const int half = (u & 1) ^ ((pc >> 3) & 1);  // stored half -> channel half
            const int sy = py0 + pr, sx = px0 + pc;
            const bool ok = (u < A_UNITS) & (sy >= 0) & (sy < H) & (sx >= 0) & (sx < W);
            r.aoff[k] = ok ? ((sy * W + sx) * cin_p + half * 8) * 2 : kOOB;
        }
        return r;
    };

    // issue the direct-to-LDS loads of stage st of tile tl into buffer buf:
    // loads k in [k0, k1) of this wave (patch loads come first)
    auto issue = [&](const Tile &tl, int st, int buf, int k0, int k1) __attribute__((always_inline)) {
        u32x4 *base = lds + buf * STAGE;
#pragma unroll
        for (int k = k0; k < k1; ++k) {
            const int ii = wave + NW * k;
            if (ii < A_INSTR) {
                const int off = tl.aoff[k] + st * CK * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(a_src, (lds_void *)(base + ii * 64), 16, off, 0, 0, 0);
            } else if (ii < T_INSTR) {
                const int jj = ii - A_INSTR;
                const int tap = (jj * 64) / (2 * BN);
                const int rem = jj * 64 - tap * (2 * BN);  // first (n, half) unit of this load
                const int soff = (st * b_stage + tap * cout_p * CK + rem * 8) * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(b_src, (lds_void *)(base + A_PAD + jj * 64), 16, tl.b_lane,
                                                         soff, 0, 0);
            }
        }
    };

    const int ar0 = G::row0(wm);
    const int nst = cin_p / CK;
    const int wh = fh ^ ((fx >> 3) & 1);  // stored half of this lane's weight fragment

    // fragment loads: the patch rows tap column dx reads, and tap (dy, dx)'s
    // weight fragments
    auto load_a = [&](const u32x4 *sA, int dx, half8 *af) __attribute__((always_inline)) {
        const int pc = G::pcol(fx, dx);
        const int ph = fh ^ ((pc >> 3) & 1);
#pragma unroll
        for (int a = 0; a < AROWS; ++a) af[a] = __builtin_bit_cast(half8, sA[((ar0 + a) * PW + pc) * 2 + ph]);
    };
    auto load_b = [&](const u32x4 *sB, int tap, half8 *bf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = __builtin_bit_cast(half8, sB[(tap * BN + wn * (BN / WN) + j * 32 + fx) * 2 + wh]);
    };

    if (NORM && tid < BN) gam[tid] = p.ngamma[tid];  // visible after the first barrier
    Tile cur = make_tile(t);
    issue(cur, 0, 0, 0, PER_WAVE);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    int gs = 0;  // stages run so far: stage gs sits in buffer gs & 1
    for (; t < t_end; t += t_step) {
        const bool has_next = can_walk<MODE, BN, NORM>() && t + t_step < t_end;
        const Tile nxt = make_tile(has_next ? t + t_step : t);

        f32x16 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        for (int st = 0; st < nst; ++st, ++gs) {
            const int buf = gs & 1;
            const u32x4 *sA = lds + buf * STAGE;
            const u32x4 *sB = sA + A_PAD;
            // the loads issued during this stage: the tile's next stage, or
            // after its last stage the next tile's first
            const bool last = st + 1 == nst;
            const bool do_issue = !last || has_next;
            const Tile &src = last ? nxt : cur;
            const int sst = last ? 0 : st + 1;
            // nine tap groups g = 3 dx + dy; each prefetches the next group's
            // weight fragments (and, at the last dy of a column, the next
            // column's patch fragments) before its MFMAs, so the LDS latency
            // hides behind them
            half8 af[2][AROWS], bf[2][FN];
            load_a(sA, 0, af[0]);
            load_b(sB, 0, bf[0]);
#pragma unroll
            for (int g = 0; g < 9; ++g) {
                const int dx = g / 3, dy = g % 3;
                // the next stage's loads, spread over the first DG tap groups so
                // the waves go straight to their MFMAs after the barrier and
                // the last loads still have two groups' time to land
                if (do_issue && g < DG)
                    issue(src, sst, buf ^ 1, (g * PER_WAVE + DG - 1) / DG, ((g + 1) * PER_WAVE + DG - 1) / DG);
                if (g + 1 < 9) {
                    const int gn = g + 1;
                    load_b(sB, (gn % 3) * 3 + gn / 3, bf[gn & 1]);
                    if (dy == 2) load_a(sA, dx + 1, af[(dx + 1) & 1]);
                }
                // keep the prefetch ahead of this group's MFMAs
                __builtin_amdgcn_sched_barrier(0);
                const half8 *a = af[dx & 1];
                const half8 *b = bf[g & 1];
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[G::arow(i, dy)], b[j], acc[i][j], 0, 0, 0);
            }
            // the next stage has landed (own loads) and every wave is done with
            // this one (barrier)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        const int y0 = cur.y0, x0 = cur.x0, n0 = cur.n0;

    // epilogue through LDS: accumulator element (i, j, r) of lane l is tile
    // pixel (4 wm + i, 8 (r / 4) + 4 (l / 32) + r % 4), channel
    // wn BN/2 + 32 j + l % 32. Pass q stages tile rows {q, 4 + q, 8 + q,
    // 12 + q} (wave row i = q of the four wave row groups) as [4][TW][BN]
    // f32 (pixel pitch SP); then every thread writes 16 contiguous bytes, so each tile row
    // leaves as one run of TW * BN * 4 bytes (contiguous when BN is the
    // output row width).
    // With a next tile its first stage is landing in the other buffer:
    // stage in the last stage's buffer only (the launcher keeps tiles too
    // wide for one buffer to one tile per workgroup).
    const float osc = p.oscale;
    static_assert(!(ACC && NORM), "the fused norm does not accumulate");
    float *stg = reinterpret_cast<float *>(lds + (has_next ? ((gs - 1) & 1) * STAGE : 0));
    float bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = p.bias ? p.bias[n0 + wn * (BN / WN) + j * 32 + fx] : 0.f;
    float *out = reinterpret_cast<float *>(p.c);
    // GroupNorm statistics: a thread's pieces all hold channel quad tid % 16
    // (pieces tid + NT k, 16 quads per 64-channel pixel row), so one group
    GnAcc gacc;
    const bool gn_live = GNS && (n0 + 4 * (tid & 15)) < p.gn_creal;
#pragma unroll
    for (int q = 0; q < FM; ++q) {
#pragma unroll
    for (int h = 0; h < 4 / RS; ++h) {
        constexpr int V4 = RS * TW * BN / 4;  // 16-byte pieces staged per pass
        constexpr int NPT = (V4 + NT - 1) / NT;  // pieces per thread
        // pass (q, h): wave row groups h RS .. h RS + RS - 1 stage their row q
        if (wm / RS == h) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int px = (r >> 2) * 8 + fh * 4 + (r & 3);
                    stg[((wm % RS) * TW + px) * SP + wn * (BN / WN) + j * 32 + fx] = osc * acc[q][j][r] + bv[j];
                }
        }
        // an accumulating pass loads the stream values it adds to all at
        // once, under the staging barrier: one piece's load after the
        // previous piece's store (the compiler cannot tell they never
        // overlap) waited a full memory round trip each
        // (with 8 waves a thread has only half the pieces, and loading them
        // in the loop below measured faster; with the GroupNorm statistics
        // as well, the 4-wave kernel has no registers left for them)
        constexpr bool HOIST = ACC && NW == 4 && !GNS;
        f32x4 res[HOIST ? NPT : 1];
        if constexpr (HOIST) {
#pragma unroll
            for (int k = 0; k < NPT; ++k) {
                // piece tid + NT k: staged row, pixel and channel as below
                const int e = (tid + NT * k) * 4;
                const int oy = y0 + FM * (h * RS + e / (TW * BN)) + q, ox = x0 + (e / BN) % TW, ch = e % BN;
                const bool in = oy < Hout && ox < Wout;
                res[k] = in ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(
                                  out + ((int64_t)oy * Wout + ox) * p.ldc + n0 + ch))
                            : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        __syncthreads();
        static_assert(V4 % NT == 0, "whole pieces per thread");
        // piece v: its staged value (plus the stream value r when
        // accumulating) to the f32 output, the guarded cast, the statistics
        auto emit = [&](int v, const f32x4 &r) __attribute__((always_inline)) {
            const int e = v * 4;
            const int wr = e / (TW * BN);  // staged row: tile row FM (h RS + wr) + q
            const int px = (e / BN) % TW;
            const int ch = e % BN;
            const int oy = y0 + FM * (h * RS + wr) + q, ox = x0 + px;
            if (oy < Hout && ox < Wout) {
                float4 val = (SP == BN) ? reinterpret_cast<const float4 *>(stg)[v]
                                        : *reinterpret_cast<const float4 *>(stg + (wr * TW + px) * SP + ch);
                float *dst = out + ((int64_t)oy * Wout + ox) * p.ldc + n0 + ch;
                if constexpr (ACC) {
                    const f32x4 o = HOIST ? r : *reinterpret_cast<const f32x4 *>(dst);
                    val.x += o[0];
                    val.y += o[1];
                    val.z += o[2];
                    val.w += o[3];
                }
                if constexpr (GNS) {
                    if (gn_live) gacc.fold4(val);
                }
                // streaming store: the tile is written once and not read
                // again by this kernel
                if (p.write_out)
                    __builtin_nontemporal_store(f32x4{val.x, val.y, val.z, val.w}, reinterpret_cast<f32x4 *>(dst));
                if (!NORM && p.yg) {
                    const float gs = p.gscale;
                    half4v hv;
                    hv[0] = (_Float16)(val.x * gs);
                    hv[1] = (_Float16)(val.y * gs);
                    hv[2] = (_Float16)(val.z * gs);
                    hv[3] = (_Float16)(val.w * gs);
                    *reinterpret_cast<half4v *>(p.yg + ((int64_t)oy * Wout + ox) * p.ldc + n0 + ch) = hv;
                }
            }
        };
        if ((!NORM && p.yg) || p.write_out) {
            if constexpr (HOIST) {
#pragma unroll
                for (int k = 0; k < NPT; ++k) emit(tid + NT * k, res[k]);
            } else {
#pragma unroll
                for (int v = tid; v < V4; v += NT) emit(v, f32x4{0.f, 0.f, 0.f, 0.f});
            }
        }
        if constexpr (NORM) {
            // the staged RS x TW pixels' RMS_norm: TPP consecutive lanes per
            // pixel, CPL channels each (the tile holds every channel: BN = N)
            constexpr int TPP = NT / (RS * TW);
            constexpr int CPL = BN / TPP;
            constexpr int NV = CPL / 4;  // float4 per lane
            static_assert(CPL == 32 || CPL == 16, "16 or 32 channels per lane");
            const int pi = tid / TPP, q4 = tid % TPP, cb = q4 * CPL;
            const int wr = pi / TW, px = pi % TW;
            const float4 *sv = reinterpret_cast<const float4 *>(stg + (wr * TW + px) * SP + cb);
            float4 v[NV];  // v[k] holds channels cb + 4 k .. + 3
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                v[k] = sv[k];
                ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
            }
#pragma unroll
            for (int off = TPP / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, TPP);
            const float inv = sqrtf((float)p.norm_c) / fmaxf(sqrtf(ss), p.norm_eps);
            const int oy = y0 + FM * (h * RS + wr) + q, ox = x0 + px;
            if (oy < Hout && ox < Wout) {
                const float4 *g4 = reinterpret_cast<const float4 *>(gam + cb);
                _Float16 *dst = p.ny + ((int64_t)oy * Wout + ox) * BN + cb;
                // SiLU as y * rcp(1 + exp(-y)) with the hardware reciprocal
                // (~1 ulp): the epilogue has no partner workgroup to hide
                // behind, and a full-precision divide is about ten
                // instructions. Without SiLU the factor is rcp(1) = 1 exactly.
                const bool silu = p.norm_silu != 0;
#pragma unroll
                for (int k = 0; k < NV; k += 2) {
                    const int u = k;  // even: 8 channels, 16-byte aligned
                    float o[8] = {v[k].x, v[k].y, v[k].z, v[k].w, v[k + 1].x, v[k + 1].y, v[k + 1].z, v[k + 1].w};
                    const float4 ga = g4[u], gb = g4[u + 1];
                    const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
                    half8 h;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float y = o[e] * inv * gm[e];
                        const float ex = silu ? __expf(-y) : 0.f;
                        h[e] = (_Float16)(y * __builtin_amdgcn_rcpf(1.0f + ex));
                    }
                    *reinterpret_cast<half8 *>(dst + 4 * u) = h;
                }
            }
        }
        __syncthreads();
    }
    }
    if constexpr (GNS) {
        // the tile's partial per group: lanes l, l ^ 16, l ^ 32, l ^ 48 hold
        // one channel quad, lanes of consecutive quads one group; then the
        // waves' partials through LDS
        const int qpg = p.gn_cpg >> 2;
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1)
            gacc.merge(__shfl_xor(gacc.n, o), __shfl_xor(gacc.m, o), __shfl_xor(gacc.q, o));
        for (int o = 1; o < qpg; o <<= 1)
            gacc.merge(__shfl_xor(gacc.n, o), __shfl_xor(gacc.m, o), __shfl_xor(gacc.q, o));
        if (lane < 16 && lane % qpg == 0) {
            float *e = gns + (wave * 16 + lane / qpg) * 3;
            e[0] = gacc.n;
            e[1] = gacc.m;
            e[2] = gacc.q;
        }
        __syncthreads();
        const int g = n0 / p.gn_cpg + tid;
        if (tid < 64 / p.gn_cpg && g * p.gn_cpg < p.gn_creal) {
            GnAcc t0;
            for (int w = 0; w < NW; ++w) t0.merge(gns[(w * 16 + tid) * 3], gns[(w * 16 + tid) * 3 + 1], gns[(w * 16 + tid) * 3 + 2]);
            const int pt = t / n_tiles;  // the pixel tile
            float *o = p.gn_part + ((int64_t)g * p.gn_nchunk + pt) * 3;
            o[0] = t0.n;
            o[1] = t0.m;
            o[2] = t0.q;
        }
        // (the next tile's partials reuse gns only after its stages' barriers)
    }
    cur = nxt;
    }
}

// workgroups resident at once: the compute units times the workgroups one
// holds (queried once per device)
int resident_slots(int per_cu)
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        cus[dev] = n;
    }
    return cus[dev] * per_cu;
}

template <int MODE, int BN, int NW, bool NORM = false, bool GNS = false>
void launch_t(const IgemmArgs &a, hipStream_t s)
{
    const int Hout = (MODE == kConv3x3Up2) ? 2 * a.H : a.H;
    const int Wout = (MODE == kConv3x3Up2) ? 2 * a.W : a.W;
    const int tiles = ((Hout + TH - 1) / TH) * ((Wout + TW - 1) / TW) * (a.N / BN);
    // where a workgroup can walk several tiles: as many workgroups as are
    // resident at once (8 waves per compute unit), a multiple of 8 for the
    // XCD schedule; else one tile each
    int grid = tiles;
    if (can_walk<MODE, BN, NORM>()) {
        const int slots = resident_slots(8 / NW) & ~7;
        if (slots > 0 && slots < tiles) grid = slots;
    }
    if constexpr (!NORM) {
        if (a.accumulate) {
            hipLaunchKernelGGL((k_conv_halo<MODE, BN, NW, NORM, GNS, true>), dim3(grid), dim3(64 * NW), 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((k_conv_halo<MODE, BN, NW, NORM, GNS>), dim3(grid), dim3(64 * NW), 0, s, a);
}

}  // namespace

void launch_conv_halo(int mode, const IgemmArgs &a, hipStream_t s)
{
    if (a.M <= 0) return;
    // (GroupNorm statistics are gathered by this kernel's epilogue only)
    if (!a.gn_part && conv_ws_supported(mode, a)) {
        launch_conv_ws(mode, a, s);
        return;
    }
    if (a.ngamma) {
        // the fused RMS_norm needs every channel of a pixel in one tile
        if (mode == kConv3x3) {
            if (a.N == 128) launch_t<kConv3x3, 128, 8, true>(a, s);
            else launch_t<kConv3x3, 64, 4, true>(a, s);
        } else {
            if (a.N == 128) launch_t<kConv3x3Up2, 128, 8, true>(a, s);
            else launch_t<kConv3x3Up2, 64, 4, true>(a, s);
        }
        return;
    }
    // 64-channel tiles (128-channel tiles measured slower on every shape of
    // the decoder), on 4 waves with two workgroups per CU, so one's epilogue
    // overlaps the other's MFMAs. With no more tiles than CUs (one
    // workgroup per CU anyway) the plain conv splits a tile over 8 waves
    // (4 rows x 32 channels each: two waves per SIMD instead of one).
    if (mode == kConv3x3) {
        const int tiles = ((a.H + TH - 1) / TH) * ((a.W + TW - 1) / TW) * (a.N / 64);
        const int cus = resident_slots(1);
        const bool eight = cus > 0 && tiles <= cus;
        if (a.gn_part) {
            if (eight) launch_t<kConv3x3, 64, 8, false, true>(a, s);
            else launch_t<kConv3x3, 64, 4, false, true>(a, s);
        } else if (eight) {
            launch_t<kConv3x3, 64, 8>(a, s);
        } else {
            launch_t<kConv3x3, 64, 4>(a, s);
        }
    } else if (a.gn_part) {
        launch_t<kConv3x3Up2, 64, 4, false, true>(a, s);
    } else {
        launch_t<kConv3x3Up2, 64, 4>(a, s);
    }
}

int conv_gn_chunks(int mode, int H, int W)
{
    const int Hout = (mode == kConv3x3Up2) ? 2 * H : H;
    const int Wout = (mode == kConv3x3Up2) ? 2 * W : W;
    return ((Hout + TH - 1) / TH) * ((Wout + TW - 1) / TW);
}

bool conv_gn_stats_supported(int cout_p, int c_real, int groups)
{
    if (groups <= 0 || c_real <= 0 || c_real > cout_p || c_real % groups) return false;
    const int cpg = c_real / groups;
    return cout_p % 64 == 0 && cpg % 4 == 0 && 64 % cpg == 0;
}

}  // namespace ig
