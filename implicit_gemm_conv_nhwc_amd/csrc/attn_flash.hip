// The mid attention's core in one pass over the keys, for gfx950:
// out[i] = f16( sum_j softmax_j(q_i . k_j / sqrt(C)) v_j + bv ),  C = 512.
//
// Page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs", `attention`: S =
// Q.K^T / sqrt(C) in f32, a row softmax to f16 P, O = P.V, V's bias added
// after the product; page "cortiq-engine 0.7.6, src/vae.rs",
// `AttnBlock::apply`, for the max-subtracted softmax. The pages store S
// (and P) per query chunk; here neither leaves the chip: the row softmax
// is taken online (Milakov and Gimelshein's running max and sum, as in
// FlashAttention), each key block's scores turning into f16 weights in
// registers that feed the P.V product directly.
//
// Design:
//  * a workgroup of 4 wave64s (one per SIMD) owns 128 queries, a wave 32 of
//    them. A wave keeps its queries' 512-wide rows in registers as the B
//    operand of v_mfma_f32_32x32x16_f16 (128 VGPRs) and its output rows as
//    16 f32 accumulator tiles (256 registers);
//  * keys advance 32 per block: the block's K rows (32 x 512) and V^T
//    columns (512 x 32) stream into double-buffered LDS by direct-to-LDS
//    buffer loads (rows past the buffers read zero);
//  * scores are computed transposed, S^T = K . Q^T (keys as MFMA rows), and
//    the output as O^T = V^T . P^T: a lane then holds one query's scores
//    and one query's output columns, so the softmax needs no cross-lane
//    traffic beyond the lane pair sharing a query, and a rescale is a
//    per-lane multiply. MFMA row r reads key r with bits 2 and 3 swapped,
//    which puts each lane's 16 scores in the key order of the P.V
//    operand (8 consecutive keys per K step);
//  * the running max is raised only when a block's max exceeds it by more
//    than 2^8 in the exponential: the weights then stay <= 256 (exact in
//    f16's range) and the rescale of the 256 output registers is rare;
//  * LDS rows are swizzled (K: 16-byte unit u of key row k at u ^ (k & 15);
//    V^T: unit u of column c at u ^ ((c >> 2) & 3)) so every fragment read
//    touches 16 distinct bank groups per pass;
//  * when the queries alone give fewer workgroups than the chip has CUs,
//    the keys are split into ranges whose partial (max, sum, O) are merged
//    by a second kernel.
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

constexpr int C = 512;             // head width
constexpr int NT = 256;            // 4 waves
constexpr int BQ = 128;            // queries per workgroup
constexpr int BK = 32;             // keys per block
constexpr int KS = C / 16;         // K steps of the score product
constexpr int CT = C / 32;         // output column tiles
constexpr int KU = BK * C / 8;     // 16-byte units of a K block (2048)
constexpr int VU = C * BK / 8;     // units of a V^T block (2048)
constexpr int STAGE = KU + VU;     // 64 KB
constexpr int LPW = KU / 64 / 4;   // loads per wave per block, K and V^T each (8)
constexpr float kHeadroom = 8.f;   // log2 of the largest weight before a rescale
constexpr float kNegBig = -1e30f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// MFMA row -> key within a block: bits 2 and 3 swapped
__device__ __forceinline__ int key_of_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// o *= alpha in place in the accumulation registers (rare: when a running
// max is raised). The products are written through VALU copies; the waits
// cover the MFMA results being read and the rewritten registers feeding
// the next MFMAs.
__device__ __forceinline__ void rescale(f32x16 (&o)[CT], float alpha)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = o[c][i], t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t)
                         : "v"(alpha));
            o[c][i] = x;
        }
    }
    asm volatile("s_nop 7" ::: "memory");
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_flash(FlashArgs p)
{
    __shared__ __attribute__((aligned(16))) u32x4 lds[2 * STAGE];

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
    const __amdgpu_buffer_rsrc_t k_src = make_rsrc(p.k, (uint32_t)((uint64_t)p.ld * C * 2));
    const __amdgpu_buffer_rsrc_t v_src = make_rsrc(p.vt, (uint32_t)((uint64_t)C * p.ld * 2));

    // this wave's queries: lane (r, h) holds q[q0 + r][16 s + 8 h .. + 7]
    half8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qf[s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
                                              q_src, ((q0 + r) * C + 16 * s + 8 * h) * 2, 0, 0));

    // loads: the wave's i-th K load fills LDS key row kr = wave + 4 i (one
    // row = 64 units, lane = stored unit); its i-th V^T load fills columns
    // 16 kc .. 16 kc + 15 (kc = wave + 4 i), 4 units each
    auto issue = [&](int blk, int buf) __attribute__((always_inline)) {
        u32x4 *base = lds + buf * STAGE;
        const int kbase = blk * BK * C * 2;  // bytes
        const int vbase = blk * BK * 2;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int kr = wave + 4 * i;
            const int u = lane ^ (kr & 15);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(k_src, (lds_void *)(base + kr * 64), 16,
                                                     (kr * C + 8 * u) * 2, kbase, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int kc = wave + 4 * i;
            const int c = 16 * kc + (lane >> 2);
            const int u = (lane & 3) ^ ((c >> 2) & 3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(v_src, (lds_void *)(base + KU + kc * 64), 16,
                                                     c * p.ld * 2 + 16 * u, vbase, 0, 0);
        }
    };

    // fragment read offsets (units): K step s = 8 a + b reads unit
    // krow * 64 + ((2 s + h) ^ (krow & 15)) = krow * 64 + 16 a + ((2 b + h) ^ (krow & 15))
    const int krow = key_of_row(r);
    int koff[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) koff[b] = krow * 64 + ((2 * b + h) ^ (krow & 15));
    // V^T tile ct, K step t: column 32 ct + r, unit (2 t + h) ^ ((r >> 2) & 3)
    int voff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) voff[t] = KU + 4 * r + ((2 * t + h) ^ ((r >> 2) & 3));

    f32x16 o[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) o[c] = f32x16{};
    float mrun = kNegBig, lsum = 0.f;
    const float sl2 = p.scale_log2;

    if (b0 < b1) issue(b0, 0);
    for (int blk = b0; blk < b1; ++blk) {
        const int buf = (blk - b0) & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (blk + 1 < b1) issue(blk + 1, buf ^ 1);
        const u32x4 *sb = lds + buf * STAGE;

        // S^T = K . Q^T over the 512 channels, two accumulation chains; the
        // fragments of the next 4 K steps are read while the current 4 run
        // (the scheduling barriers keep the reads from being hoisted
        // further, which would exhaust the registers)
        f32x16 sa = f32x16{}, sc = f32x16{};
        {
            half8 kc[4], kn[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) kc[i] = __builtin_bit_cast(half8, sb[koff[i]]);
#pragma unroll
            for (int g = 0; g < KS / 4; ++g) {
                if (g + 1 < KS / 4) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s2 = 4 * (g + 1) + i;
                        kn[i] = __builtin_bit_cast(half8, sb[koff[s2 & 7] + 16 * (s2 >> 3)]);
                    }
                }
                sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(kc[0], qf[4 * g], sa, 0, 0, 0);
                sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kc[1], qf[4 * g + 1], sc, 0, 0, 0);
                sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(kc[2], qf[4 * g + 2], sa, 0, 0, 0);
                sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kc[3], qf[4 * g + 3], sc, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) kc[i] = kn[i];
            }
        }
        // lane (r, h) register j: query q0 + r, key 8 h + j (j < 8) or
        // 16 + 8 h + (j - 8) of the block
        float t[16];
        float bm = kNegBig;
        const int kb = blk * BK;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            t[j] = (sa[j] + sc[j]) * sl2;
            const int key = kb + (j < 8 ? 8 * h + j : 16 + 8 * h + (j - 8));
            if (kb + BK > p.m && key >= p.m) t[j] = kNegBig;
            bm = fmaxf(bm, t[j]);
        }
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const bool raise = bm > mrun + kHeadroom;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float alpha = raise ? __builtin_amdgcn_exp2f(mrun - bm) : 1.f;
            if (raise) mrun = bm;
            lsum *= alpha;
            rescale(o, alpha);
        }
        half8 pk[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float w = __builtin_amdgcn_exp2f(t[j] - mrun);
            lsum += w;
            pk[j >> 3][j & 7] = (_Float16)w;
        }
        // O^T += V^T . P^T, two column tiles (4 fragments) at a time
        {
            half8 vc[4], vn[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) vc[i] = __builtin_bit_cast(half8, sb[voff[i & 1] + 128 * (i >> 1)]);
#pragma unroll
            for (int g = 0; g < CT / 2; ++g) {
                if (g + 1 < CT / 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vn[i] = __builtin_bit_cast(half8, sb[voff[i & 1] + 128 * (2 * (g + 1) + (i >> 1))]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[2 * g + (i >> 1)] =
                        __builtin_amdgcn_mfma_f32_32x32x16_f16(vc[i], pk[i & 1], o[2 * g + (i >> 1)], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) vc[i] = vn[i];
            }
        }
    }

    // lane (r, h) holds output columns 32 c + 8 (j / 4) + 4 h + j % 4 of query q0 + r
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const int q = q0 + r;
    if (q >= p.m) return;
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
            p.ml[((int64_t)sp * p.m + q) * 2] = mrun;
            p.ml[((int64_t)sp * p.m + q) * 2 + 1] = ltot;
        }
    }
}

// merge the key ranges' partial results of one query row:
// out = f16( sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s + bv )
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

// key ranges: enough workgroups to cover the chip, each range >= 8 blocks
void flash_split(int m, int &nsplit, int &bps)
{
    const int nqb = (m + BQ - 1) / BQ;
    const int nblocks = (m + BK - 1) / BK;
    int ns = (256 + nqb - 1) / nqb;
    const int cap = nblocks / 8 > 1 ? nblocks / 8 : 1;
    if (ns > cap) ns = cap;
    bps = (nblocks + ns - 1) / ns;
    nsplit = (nblocks + bps - 1) / bps;
}

}  // namespace

bool flash_supported(int m, int ld, int c) { return c == C && m > 0 && ld >= ((m + BK - 1) / BK) * BK && ld % 8 == 0; }

size_t flash_workspace_bytes(int m)
{
    int ns, bps;
    flash_split(m, ns, bps);
    if (ns == 1) return 0;
    return (size_t)ns * m * (C + 2) * sizeof(float) + 256;
}

void launch_flash(FlashArgs a, void *ws, hipStream_t s)
{
    if (a.m <= 0) return;
    flash_split(a.m, a.nsplit, a.bps);
    if (a.nsplit > 1) {
        a.opart = reinterpret_cast<float *>(ws);
        a.ml = a.opart + (int64_t)a.nsplit * a.m * C;
    }
    const int nqb = (a.m + BQ - 1) / BQ;
    hipLaunchKernelGGL(k_flash, dim3(nqb * a.nsplit), dim3(NT), 0, s, a);
    if (a.nsplit > 1) hipLaunchKernelGGL(k_flash_merge, dim3(a.m), dim3(128), 0, s, a);
}

}  // namespace ig
