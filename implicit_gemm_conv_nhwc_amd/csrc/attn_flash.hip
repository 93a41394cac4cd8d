// The mid attention's core in one pass over the keys, for gfx950:
// out[i] = f16( sum_j softmax_j(q_i . k_j / sqrt(C)) v_j + bv ),
// C = 128, 256, 384 or 512.
//
// Page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs", `attention`: S =
// Q.K^T / sqrt(C) in f32, a row softmax to f16 P, O = P.V, V's bias added
// after the product; page "cortiq-engine 0.7.6, src/vae.rs",
// `AttnBlock::apply`, for the max-subtracted softmax. The pages store S
// (and P) per query chunk; here neither leaves the chip: the row softmax
// is accumulated block by block (the sums of exp(s - ref) and of the
// weighted V rows, normalised at the end, as in Milakov and Gimelshein's
// online softmax and FlashAttention), each key block's scores turning into
// f16 weights in registers that feed the P.V product directly.
//
// Design:
//  * a workgroup of 4 wave64s (one per SIMD) owns 128 queries, a wave 32 of
//    them. A wave keeps its queries' C-wide rows in registers as the B
//    operand of v_mfma_f32_32x32x16_f16 (C / 4 VGPRs: 128 at C = 512) and
//    its output rows as C / 32 f32 accumulator tiles (C / 2 registers);
//  * keys advance 32 per block: the block's K rows (32 x C) and V^T
//    columns (C x 32) stream into double-buffered LDS by direct-to-LDS
//    buffer loads (rows past the buffers read zero);
//  * scores are computed transposed, S^T = K . Q^T (keys as MFMA rows), and
//    the output as O^T = V^T . P^T: a lane then holds one query's scores
//    and one query's output columns, so the softmax needs no cross-lane
//    traffic beyond the lane pair sharing a query. MFMA row r reads key r
//    with bits 2 and 3 swapped,
//    which puts each lane's 16 scores in the key order of the P.V
//    operand (8 consecutive keys per K step);
//  * the weights are taken relative to a reference max per query fixed for
//    the whole pass (the first key block's max) rather than a running max,
//    so the 256 output registers are never rescaled inside the loop: a
//    weight is at most 2^15, within f16's range, unless a later block's max
//    exceeds the reference by more than that; then the workgroup runs a
//    second pass with the range's true max as the reference;
//  * software pipeline: an iteration computes block b's scores, then runs
//    block b - 1's P.V product while it turns block b's scores into
//    weights, so the softmax's VALU work overlaps the MFMAs of a single
//    wave per SIMD; the score MFMAs are inline asm with the accumulator
//    pinned to VGPRs, keeping every AGPR for the output;
//  * at C = 512 a K row (64 units of 16 bytes) is one wave's load and
//    rows are padded to 65 units in LDS; narrower rows are packed, a load
//    spanning several of them, and unit u of key row j sits at
//    u ^ (j mod 16) within its group of 16. V^T units are swizzled too
//    (unit u of column c at u ^ ((c >> 2) & 3)). Either way every fragment
//    read touches 16 distinct bank groups per pass;
//  * when the queries alone give fewer workgroups than the chip has CUs,
//    the keys are split into ranges whose partial (max, sum, O) are merged
//    by a second kernel;
//  * the direct-to-LDS loads are issued as asm one per two score MFMAs:
//    a vector-memory issue holds up the single wave of its SIMD for a
//    while, and next to an MFMA that time is hidden.
#include <math.h>

#include "ig_internal.h"

namespace ig {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NT = 256;            // 4 waves
constexpr int BQ = 128;            // queries per workgroup
constexpr int BK = 32;             // keys per block
constexpr int PD = 3;              // fragment reads in flight ahead of the MFMAs
// the geometry at head width C (a multiple of 128, at most 512)
template <int C>
struct FGeo {
    static_assert(C % 128 == 0 && C >= 128 && C <= 512, "head width");
    static constexpr int KS = C / 16;            // K steps of the score product
    static constexpr int CT = C / 32;            // output column tiles
    static constexpr int KUR = C / 8;            // 16-byte units of a K row
    static constexpr bool KPAD = C == 512;       // a K row per wave load, rows padded
    static constexpr int KROW = KPAD ? KUR + 1 : KUR;  // LDS units per K row
    static constexpr int KBUF = BK * KROW;       // LDS units per K buffer
    static constexpr int VU = C * BK / 8;        // units of a V^T block
    static constexpr int LPW = BK * KUR / 64 / 4;  // loads per wave per block, K and V^T each (C / 64)
    static constexpr int NH = CT / 2;            // softmax hooks per P.V phase
};
constexpr float kHeadroom = 15.f;  // log2 of the largest weight (f16 holds up to 2^16)
constexpr float kNegBig = -1e30f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// A buffer descriptor as four SGPRs (raw buffer: stride 0, num_records
// bytes, the same flags as make_rsrc), for the asm loads below.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 sgpr_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// A 16-byte-per-lane direct-to-LDS buffer load written as asm: the loads
// stream the next blocks into LDS while the current ones are read, and the
// kernel orders them itself (s_waitcnt vmcnt(0) and a barrier before a
// block is read). Seen as builtins, every LDS read after such a load would
// get a wait for it.
__device__ __forceinline__ void dma16(i32x4 rsrc, const void *lds_dst, int voff, int soff)
{
    const unsigned addr = (unsigned)(uintptr_t)lds_dst;
    unsigned saved;
    // M0 holds the LDS address; its previous value is restored
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(addr)), "v"(voff), "s"(rsrc),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory");
}

// max(a, b, c) of finite scores, as one v_max3_f32 (fmaxf on values the
// compiler cannot prove canonical adds a canonicalizing max per operand)
__device__ __forceinline__ float max3_raw(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// MFMA row -> key within a block: bits 2 and 3 swapped
__device__ __forceinline__ int key_of_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// The score accumulation runs as inline-asm MFMAs whose accumulator is
// pinned to VGPRs, so the 256 output accumulators keep the AGPRs to
// themselves. A chain's MFMAs read their predecessor's result as SrcC with
// the same registers (no wait states needed); the first starts from zero
// (no SrcC read); the last pads 16 wait states so the VALU may read its
// result right after.
__device__ __forceinline__ void mfma_first(f32x16 &acc, half8 a, half8 b)
{
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16 &acc, half8 a, half8 b)
{
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_last(f32x16 &acc, half8 a, half8 b)
{
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7" : "+v"(acc) : "v"(a), "v"(b));
}

template <int C>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_flash(FlashArgs p)
{
    using G = FGeo<C>;
    constexpr int KS = G::KS, CT = G::CT, KUR = G::KUR, KROW = G::KROW, KBUF = G::KBUF, VU = G::VU, LPW = G::LPW;
    __shared__ __attribute__((aligned(16))) u32x4 lds[2 * (KBUF + VU)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, h = lane >> 5;

    // workgroups are dealt round robin to the 8 XCDs: give each XCD a
    // contiguous run of (key range, query block) pairs, so the workgroups
    // of an XCD stream the same K / V^T blocks through its L2
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int nqb = (p.m + BQ - 1) / BQ;
    const int sp = bid / nqb, qb = bid % nqb;
    const int nblocks = (p.m + BK - 1) / BK;
    const int b0 = sp * p.bps;
    const int b1 = (b0 + p.bps) < nblocks ? (b0 + p.bps) : nblocks;
    const int q0 = qb * BQ + wave * 32;

    const __amdgpu_buffer_rsrc_t q_src = make_rsrc(p.q, (uint32_t)((uint64_t)p.ld * C * 2));
    const i32x4 k_src = sgpr_rsrc(p.k, (uint32_t)((uint64_t)p.ld * C * 2));
    const i32x4 v_src = sgpr_rsrc(p.vt, (uint32_t)((uint64_t)C * p.ld * 2));

    // this wave's queries: lane (r, h) holds q[q0 + r][16 s + 8 h .. + 7]
    half8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qf[s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
                                              q_src, ((q0 + r) * C + 16 * s + 8 * h) * 2, 0, 0));

    // LDS: two K buffers (key rows KROW units apart), then two V^T
    // buffers. At C = 512 the wave's i-th K load fills key row kr = wave +
    // 4 i (64 units from the lane's 16 bytes); narrower, it fills LDS units
    // U = (wave + 4 i) 64 + lane, unit U mod KUR of key row U / KUR, read
    // from the row's unit (U mod KUR) ^ (row mod 16). Its i-th V^T load
    // fills columns 16 kc .. 16 kc + 15 (kc = wave + 4 i), 4 units each,
    // unit u of column c at u ^ ((c >> 2) & 3). Per-lane source offsets
    // are fixed; the load index and the block move the scalar offset.
    u32x4 *const ldv = lds + 2 * KBUF;
    const int kvoff = 16 * lane;
    int kvo[G::KPAD ? 1 : LPW];
    if constexpr (!G::KPAD) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int u = (wave + 4 * i) * 64 + lane, kr = u / KUR, ku = u % KUR;
            kvo[i] = kr * C * 2 + 16 * (ku ^ (kr & 15));
        }
    }
    const int vvoff = (int)((uint32_t)(16 * wave + (lane >> 2)) * (uint32_t)p.ld * 2u +
                            16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)));
    auto issue_k = [&](int blk, int kbuf, int i) __attribute__((always_inline)) {
        if constexpr (G::KPAD) {
            const int kr = wave + 4 * i;
            dma16(k_src, lds + kbuf * KBUF + kr * KROW, kvoff, (blk * BK + kr) * C * 2);
        } else {
            dma16(k_src, lds + kbuf * KBUF + (wave + 4 * i) * 64, kvo[i], blk * BK * C * 2);
        }
    };
    auto issue_v = [&](int blk, int vbuf, int i) __attribute__((always_inline)) {
        dma16(v_src, ldv + vbuf * VU + (wave + 4 * i) * 64, vvoff, (int)((uint32_t)i * 64u * (uint32_t)p.ld * 2u + (uint32_t)blk * BK * 2u));
    };

    // fragment reads (units): K step s of MFMA row r reads key row
    // kr = key_of_row(r), unit 2 s + h: with padded rows at krd + 2 s, else
    // at kr KUR + (2 s + h) ^ (kr mod 16) = kq[s mod 8] + 16 (s / 8); 16
    // consecutive lanes hit 16 distinct bank groups. V^T tile ct, K step t:
    // column 32 ct + r, unit (2 t + h) ^ ((r >> 2) & 3)
    const int krd = key_of_row(r) * KROW + h;
    int kq[G::KPAD ? 1 : 8];
    if constexpr (!G::KPAD) {
        const int kr = key_of_row(r);
#pragma unroll
        for (int k = 0; k < 8; ++k) kq[k] = kr * KUR + ((2 * k + h) ^ (kr & 15));
    }
    auto kunit = [&](int st) __attribute__((always_inline)) {
        if constexpr (G::KPAD) return krd + 2 * st;
        else return kq[st & 7] + 16 * (st >> 3);
    };
    int voff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) voff[t] = 4 * r + ((2 * t + h) ^ ((r >> 2) & 3));

    const float sl2 = p.scale_log2;
    float ref = kNegBig, mtrue = kNegBig, bmax = kNegBig;
    bool over = false;

    // One pass over the key range: the pipeline below, then the epilogue.
    // Returns true (writing nothing) when the first pass must be redone.
    auto run = [&](const bool first) __attribute__((always_inline)) -> bool {
    f32x16 o[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) o[c] = f32x16{};
    float lsum = 0.f;

    // S^T of one block from K buffer kbuf, with hook(st) run after the MFMA
    // of K step st. Fragments are read PD steps ahead into a ring of
    // PD + 1; the scheduling barriers keep the reads from being hoisted
    // further (which would exhaust the registers).
    auto s_phase = [&](int kbuf, f32x16 &sacc, auto &&hook) __attribute__((always_inline)) {
        const u32x4 *sk = lds + kbuf * KBUF;
        half8 kf[PD + 1];
#pragma unroll
        for (int i = 0; i < PD; ++i) kf[i] = __builtin_bit_cast(half8, sk[kunit(i)]);
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            if (st + PD < KS) {
                const int s2 = st + PD;
                kf[s2 % (PD + 1)] = __builtin_bit_cast(half8, sk[kunit(s2)]);
            }
            const half8 a = kf[st % (PD + 1)];
            if (st == 0)
                mfma_first(sacc, a, qf[0]);
            else if (st + 1 < KS)
                mfma_acc(sacc, a, qf[st]);
            else
                mfma_last(sacc, a, qf[st]);
            hook(st);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // O^T += V^T . P^T from V^T buffer vbuf, with hook(g) run before the
    // products of column tiles 2 g and 2 g + 1. Fragment f = 4 g + i holds
    // column tile 2 g + (i & 1), K step i >> 1 (a tile's two K steps apart)
    auto pv_phase = [&](int vbuf, const half8 (&pk)[2], auto &&hook) __attribute__((always_inline)) {
        const u32x4 *sv = ldv + vbuf * VU;
        auto vread = [&](int f) __attribute__((always_inline)) {
            const int i = f & 3, g = f >> 2;
            return __builtin_bit_cast(half8, sv[voff[i >> 1] + 128 * (2 * g + (i & 1))]);
        };
        half8 vf[PD + 1];
#pragma unroll
        for (int f = 0; f < PD; ++f) vf[f] = vread(f);
#pragma unroll
        for (int f = 0; f < 2 * CT; ++f) {
            if (f + PD < 2 * CT) vf[(f + PD) % (PD + 1)] = vread(f + PD);
            const int i = f & 3, g = f >> 2;
            if (i == 0) hook(g);
            o[2 * g + (i & 1)] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[f % (PD + 1)], pk[i >> 1],
                                                                         o[2 * g + (i & 1)], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // softmax step g of a block whose raw scores are in sacc (lane (r, h)
    // register j: query q0 + r, key 8 h + j (j < 8) or 16 + 8 h + (j - 8)
    // of the block): the block's max of the raw scores, taken to the log2
    // domain afterwards (the scale sl2 > 0 commutes with the max), then the
    // weights 2^(t sl2 - ref) of the keys below lim. ref is the query's
    // reference max, fixed for the pass (first: the range's first block's
    // max); a block whose max exceeds it by more than the headroom marks
    // the wave for a second pass with ref = the range's max.
    auto softmax_step = [&](int g, f32x16 &t, int lim, half8 (&pk)[2], bool first) __attribute__((always_inline)) {
        if (g == 0 || g == 1) {
            if (g == 0 && lim < BK) {
                // the sequence's last, partial block: keys >= m weigh 0
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = j < 8 ? 8 * h + j : 16 + 8 * h + (j - 8);
                    if (key >= lim) t[j] = kNegBig;
                }
            }
            const int j0 = 8 * g;
            const float a = max3_raw(t[j0], t[j0 + 1], t[j0 + 2]);
            const float b = max3_raw(t[j0 + 3], t[j0 + 4], t[j0 + 5]);
            const float m = max3_raw(a, b, max3_raw(t[j0 + 6], t[j0 + 7], t[j0 + 7]));
            bmax = g == 0 ? m : max3_raw(bmax, m, m);
        } else if (g == 3) {
            const float bm = sl2 * max3_raw(bmax, __shfl_xor(bmax, 32), bmax);
            if (first) ref = bm;
            over = over || bm > ref + kHeadroom;
            mtrue = fmaxf(mtrue, bm);
        } else if (g == 4 || g == 5) {
            const int j0 = 8 * (g - 4);
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[j0 + e], sl2, -ref));
                pk[g - 4][e] = (_Float16)w[e];
            }
            lsum += ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
        }
    };

    // Pipeline: iteration blk computes block blk's scores (K(blk) in LDS),
    // then runs block blk - 1's P.V while it turns block blk's scores into
    // weights. Iteration blk loads K(blk + 1) and V^T(blk); past the
    // range's end the loads are of a clamped, valid block and never used.
    // A second pass runs only when a wave of the workgroup saw a block
    // exceed its reference max by more than the headroom (scores growing
    // by more than 2^15 in the exponential along the keys).
    const int last = nblocks - 1;
    f32x16 sacc;
    half8 pprev[2], pcur[2];
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue_k(b0, 0, i);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
        const int nk = b0 + 1 < last ? b0 + 1 : last;
        s_phase(0, sacc, [&](int st) {
            if (st % 4 == 1) issue_k(nk, 1, st / 4);
            if (st % 4 == 3) issue_v(b0, 0, st / 4);
        });
#pragma unroll
        for (int g = 0; g < 6; ++g) softmax_step(g, sacc, p.m - b0 * BK, pprev, first);
    }
    for (int blk = b0 + 1; blk < b1; ++blk) {
        const int cur = (blk - b0) & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int nk = blk + 1 < last ? blk + 1 : last;
        s_phase(cur, sacc, [&](int st) {
            if (st % 4 == 1) issue_k(nk, cur ^ 1, st / 4);
            if (st % 4 == 3) issue_v(blk, cur, st / 4);
        });
        const int lim = p.m - blk * BK;
        // the six softmax steps over the P.V phase's NH hooks: one per hook
        // where there are six or more, else spread evenly (narrow heads)
        pv_phase(cur ^ 1, pprev, [&](int g) __attribute__((always_inline)) {
            if constexpr (G::NH >= 6) {
                softmax_step(g, sacc, lim, pcur, false);
            } else {
#pragma unroll
                for (int st = (6 * g + G::NH - 1) / G::NH; st < (6 * (g + 1) + G::NH - 1) / G::NH; ++st)
                    softmax_step(st, sacc, lim, pcur, false);
            }
        });
        pprev[0] = pcur[0];
        pprev[1] = pcur[1];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    pv_phase((b1 - 1 - b0) & 1, pprev, [](int) {});
    if (first && __syncthreads_or(over)) return true;

    // lane (r, h) holds output columns 32 c + 8 (j / 4) + 4 h + j % 4 of query q0 + r
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const int q = q0 + r;
    if (q >= p.m) return false;
    if (p.nsplit == 1) {
        const float inv = 1.f / ltot;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * c + 8 * g + 4 * h;
                const f32x4 b = p.bv ? *reinterpret_cast<const f32x4 *>(p.bv + col) : f32x4{};
                half4v y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (_Float16)(o[c][4 * g + e] * inv + b[e]);
                *reinterpret_cast<half4v *>(p.out + (int64_t)q * C + col) = y;
            }
        }
    } else {
        float *op = p.opart + ((int64_t)sp * p.m + q) * C;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * c + 8 * g + 4 * h;
                *reinterpret_cast<f32x4 *>(op + col) =
                    f32x4{o[c][4 * g], o[c][4 * g + 1], o[c][4 * g + 2], o[c][4 * g + 3]};
            }
        }
        if (h == 0) {
            p.ml[((int64_t)sp * p.m + q) * 2] = ref;
            p.ml[((int64_t)sp * p.m + q) * 2 + 1] = ltot;
        }
    }
    return false;
    };

    // A second pass runs only when a wave of the workgroup saw a block
    // exceed its reference max by more than the headroom (scores growing
    // by more than 2^15 in the exponential along the keys); it takes the
    // range's max as the reference.
    if (run(true)) {
        ref = mtrue;
        run(false);
    }
}

// merge the key ranges' partial results of one query row (C / 4 threads):
// out = f16( sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s + bv )
template <int C>
__global__ __launch_bounds__(128) void k_flash_merge(FlashArgs p)
{
    const int q = blockIdx.x, t = threadIdx.x;
    float mx = kNegBig;
    for (int s = 0; s < p.nsplit; ++s) mx = fmaxf(mx, p.ml[((int64_t)s * p.m + q) * 2]);
    float den = 0.f;
    f32x4 acc = f32x4{};
    for (int s = 0; s < p.nsplit; ++s) {
        const float w = __builtin_amdgcn_exp2f(p.ml[((int64_t)s * p.m + q) * 2] - mx);
        den += w * p.ml[((int64_t)s * p.m + q) * 2 + 1];
        acc += w * *reinterpret_cast<const f32x4 *>(p.opart + ((int64_t)s * p.m + q) * C + 4 * t);
    }
    const float inv = 1.f / den;
    const f32x4 b = p.bv ? *reinterpret_cast<const f32x4 *>(p.bv + 4 * t) : f32x4{};
    half4v y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (_Float16)(acc[e] * inv + b[e]);
    *reinterpret_cast<half4v *>(p.out + (int64_t)q * C + 4 * t) = y;
}

// key ranges (at most 8, each >= 8 blocks): workgroups run one per CU in
// waves of 256, so the count is the fewest ranges whose workgroups fill
// those waves to 90% or more, else the count that fills them best (each
// range adds a partial result for the merge to read)
void flash_split(int m, int &nsplit, int &bps)
{
    const int nqb = (m + BQ - 1) / BQ;
    const int nblocks = (m + BK - 1) / BK;
    int cap = nblocks / 8 > 1 ? nblocks / 8 : 1;
    if (cap > 8) cap = 8;
    int ns = 1;
    double best = 0.0;
    for (int k = 1; k <= cap; ++k) {
        const int64_t w = (int64_t)nqb * k;
        const double fill = (double)w / (double)(((w + 255) / 256) * 256);
        if (fill > best + 1e-9) {
            best = fill;
            ns = k;
        }
        if (fill >= 0.9) break;
    }
    bps = (nblocks + ns - 1) / ns;
    nsplit = (nblocks + bps - 1) / bps;
}

template <int C>
void launch_flash_t(FlashArgs a, void *ws, hipStream_t s)
{
    flash_split(a.m, a.nsplit, a.bps);
    if (a.nsplit > 1) {
        a.opart = reinterpret_cast<float *>(ws);
        a.ml = a.opart + (int64_t)a.nsplit * a.m * C;
    }
    const int nqb = (a.m + BQ - 1) / BQ;
    hipLaunchKernelGGL(k_flash<C>, dim3(nqb * a.nsplit), dim3(NT), 0, s, a);
    if (a.nsplit > 1) hipLaunchKernelGGL(k_flash_merge<C>, dim3(a.m), dim3(C / 4), 0, s, a);
}

}  // namespace

// head widths 128, 256, 384, 512; q, k and V^T are addressed with 32-bit
// byte offsets: each stays below kConvInMaxBytes (ld < 2,096,960 rows at
// C = 512)
bool flash_supported(int m, int ld, int c)
{
    return (c == 128 || c == 256 || c == 384 || c == 512) && m > 0 && ld >= ((m + BK - 1) / BK) * BK &&
           ld % 8 == 0 && (int64_t)ld * c * 2 < kConvInMaxBytes;
}

size_t flash_workspace_bytes(int m, int c)
{
    int ns, bps;
    flash_split(m, ns, bps);
    if (ns == 1) return 0;
    return (size_t)ns * m * (c + 2) * sizeof(float) + 256;
}

void launch_flash(FlashArgs a, void *ws, hipStream_t s)
{
    if (a.m <= 0) return;
    switch (a.c) {
    case 128: launch_flash_t<128>(a, ws, s); break;
    case 256: launch_flash_t<256>(a, ws, s); break;
    case 384: launch_flash_t<384>(a, ws, s); break;
    default: launch_flash_t<512>(a, ws, s); break;
    }
}

}  // namespace ig
