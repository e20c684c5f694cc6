// Decode-attention kernels for gfx950 (CDNA4).
//
// Four kernels share one streaming routine:
//   lean_kernel      stream-K over a persistent grid with in-launch merging
//                    (xllm-io paper review of arXiv 2405.10480, §3.3-§3.5, §4.4)
//   pull_kernel      the same tile order in fixed chunks that workgroups pull
//                    from a counter (or take one each), merged by the last
//                    piece to arrive (siliconandsystems digest, "Exact softmax
//                    can be reduced in pieces")
//   split_kernel +   fixed split of every head into `splits` pieces and a
//   combine_kernel   second launch that merges them (the FlashDecoding scheme the
//                    same review describes in §2.3)
//   per_head_kernel  one workgroup per (request, head) over its whole context
//                    (the FlashAttention-2 decode mapping, §2.2)
//
// Streaming routine. A K or V row of d halves is d/8 pieces of 16 bytes. V
// rows are read whole by "lane groups" of d/8 consecutive lanes, each lane one
// piece, and each group keeps its own online-softmax state (m, l, Obar slice
// of 8 dims) over the rows it accumulates (§3.3: update the statistics per
// tile, then O_acc = P V + diag(rescale) O_acc). In long ranges K rows are
// read with another pattern -- 64 bytes of each of 16 rows per instruction,
// four lanes per row -- because K and V streamed side by side in the same
// pattern read slower (see stream_step); the four lanes of a K row add their
// partial dot products across the wave, and each wave hands its scores to its
// V lane groups through a small slice of LDS. Short ranges read K like V, by
// lane groups, for the lower latency of each step, and so do the long ranges
// of a lean or pull workgroup whose CU holds more of the launch's workgroups
// than its share (see stream_range, stream_step_rows and CuWatch). Decode
// attention has a single query row, so K
// and V elements are each used once: they go straight from HBM to registers
// with 16-byte loads and are not staged in LDS. At the end of a range the
// groups meet in LDS, where the reduction f (§3.2) folds them into one
// (m, l, Obar[d]).
//
// Epilogues run in wave 0. In the lean kernel a peer (a workgroup that holds
// a head's tiles but not its first one) publishes its (Obar, m, l) record and
// raises a flag once the record's stores have completed -- after the first
// step of its workgroup's next segment, so that the wave does not stop to
// wait for them; the head's host polls all its peers' flags at once and folds
// their records in ascending workgroup order (§3.5). The other waves meanwhile
// go on to the workgroup's next segment without waiting for wave 0's fold --
// except at a host with more than kMergeBatch peers, whose segment is its
// workgroup's last: there all four waves share the merge.
//
// Exponentials are taken base 2 with log2(e) folded into the scale; m is kept
// in log2 units inside the kernels and converted back to natural-log units
// for m_out.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace la {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ numerics

// Dot product of 8 packed halves (one 16-byte load) with the lane's q slice,
// accumulated in fp32 by the packed dot2 instructions.
template <int DT>
__device__ __forceinline__ float dot8(const uint4 k, const uint4 q) {
    float a = 0.f;
    if constexpr (DT == 0) {
        a = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.x), __builtin_bit_cast(half2_t, q.x), a, false);
        a = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.y), __builtin_bit_cast(half2_t, q.y), a, false);
        a = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.z), __builtin_bit_cast(half2_t, q.z), a, false);
        a = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.w), __builtin_bit_cast(half2_t, q.w), a, false);
    } else {
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.x), __builtin_bit_cast(bf162_t, q.x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.y), __builtin_bit_cast(bf162_t, q.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.z), __builtin_bit_cast(bf162_t, q.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.w), __builtin_bit_cast(bf162_t, q.w), a, false);
    }
    return a;
}

template <int DT>
__device__ __forceinline__ void widen2(uint32_t w, float& lo, float& hi) {
    if constexpr (DT == 0) {
        half2_t h = __builtin_bit_cast(half2_t, w);
        lo = (float)h.x;
        hi = (float)h.y;
    } else {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xffff0000u);
    }
}

// Sum over the lanes of one group: 8 lanes (d = 64) or 16 lanes (d = 128),
// all inside one DPP row. Every lane ends with the same bits because each
// step adds a pair of commuted operands.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    if constexpr (LPR == 16)
        x += __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false);  // row_mirror
    return x;
}

struct Acc {
    float m;      // running max, log2 units
    float l;      // running sum of 2^(s - m)
    float o[8];   // running unnormalised output, this lane's 8 dims
};

__device__ __forceinline__ void acc_init(Acc& a) {
    a.m = kNegInf;
    a.l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a.o[i] = 0.f;
}

template <int D>
struct Geo {
    static constexpr int LPR = D / 8;                 // lanes per row (16-byte pieces of a row)
    static constexpr int GPW = 64 / LPR;              // groups per wave
    static constexpr int NG = GPW * kWaves;           // groups per workgroup
    static constexpr int CH = NG * kRows;             // rows per step (workgroup)
    static constexpr int RW = GPW * kRows;            // rows per step (wave): 32 or 64
    static constexpr int SB = RW / 16;                // K: blocks of 16 rows per wave step
    static constexpr int KK = LPR / 4;                // K: 16-byte pieces of a row per lane
    static constexpr uint32_t RB = D * 2;             // bytes per row
};

// Kinds of step: every row valid; rows from the range end masked (the last
// step); rows before the range start masked too (the first step of a range
// whose step grid starts before it, see stream_range).
constexpr int kStepFull = 0, kStepTail = 1, kStepEdge = 2;
// Steps between two looks at how crowded the workgroup's CU is (stream_range).
constexpr int kCheckSteps = 16;
// Peer records whose loads a host wave keeps in flight at once.
constexpr int kMergeBatch = 16;

// One step reading K like V, by whole rows: each lane group (d/8 lanes) takes
// kRows rows, each lane a 16-byte piece `sub` of K and V, so one instruction
// of a wave reads GPW consecutive rows (1 KiB contiguous). Scores are summed
// within the lane group by DPP, with no LDS traffic, which keeps a step's
// latency low, and every CU request moves a whole 128-byte line.
//   WAVE_BLOCK: the step covers this wave's RW rows [kb, kb + RW); lane group
//     g = lane / LPR of the wave takes rows kb + GPW i + g -- the rows of each
//     wave and lane group are those of stream_step, so a wave may take either
//     routine for any step of a range.
//   otherwise: kb is the workgroup step's first row and lane group g of the
//     workgroup (of NG) takes rows kb + NG i + g, so the four waves read one
//     contiguous 4 KiB block per instruction (short ranges: measured 0.5 us
//     faster than per-wave blocks on 1024-token heads).
// Full steps address rows as (uniform base) + (fixed 32-bit lane offset); a
// tail step clamps rows at or past e to e-1 (never reading outside the head)
// and masks their scores to -inf; an edge step also clamps rows before lo to
// lo and masks them.
template <int DT, int D, int MODE, bool WAVE_BLOCK>
__device__ __forceinline__ void stream_step_rows(const char* __restrict__ kh,
                                                 const char* __restrict__ vh, int kb, int lo,
                                                 int e, const uint4 qv, float sl2e, Acc& acc) {
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int sub = lane % G::LPR;
    // first row of this lane group and the stride between its rows
    const int g0 = WAVE_BLOCK ? lane / G::LPR : (threadIdx.x >> 6) * G::GPW + lane / G::LPR;
    constexpr int kStride = WAVE_BLOCK ? G::GPW : G::NG;
    uint4 kr[kRows], vr[kRows];
    if constexpr (MODE == kStepFull) {
        const uint32_t off = (uint32_t)(kb + g0) * G::RB + (uint32_t)sub * 16u;
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            kr[i] = load_nt(kh + (uint64_t)(off + (uint32_t)i * kStride * G::RB));
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            vr[i] = load_nt(vh + (uint64_t)(off + (uint32_t)i * kStride * G::RB));
    } else {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            int row = min(kb + kStride * i + g0, e - 1);
            if constexpr (MODE == kStepEdge) row = max(row, lo);
            kr[i] = load_nt(kh + (uint64_t)((uint32_t)row * G::RB + (uint32_t)sub * 16u));
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            int row = min(kb + kStride * i + g0, e - 1);
            if constexpr (MODE == kStepEdge) row = max(row, lo);
            vr[i] = load_nt(vh + (uint64_t)((uint32_t)row * G::RB + (uint32_t)sub * 16u));
        }
    }
    // all 2*kRows loads of the step in flight before any is consumed
    __builtin_amdgcn_sched_barrier(0);
    float s[kRows];
    float mx = kNegInf;
    {
        // one rounding of the scaled score feeds both the max and exp2(s - m),
        // so the maximal row gets weight exactly 1
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const float x = group_sum<G::LPR>(dot8<DT>(kr[i], qv)) * sl2e;
            const int row = kb + kStride * i + g0;
            s[i] = (MODE == kStepFull || (row < e && (MODE != kStepEdge || row >= lo))) ? x : kNegInf;
            mx = fmaxf(mx, s[i]);
        }
    }
    const float mn = fmaxf(acc.m, mx);
    const float mu = (mn == kNegInf) ? 0.f : mn;   // no -inf - -inf
    const float alpha = fexp2(acc.m - mu);
    acc.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.o[i] *= alpha;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const float p = fexp2(s[r] - mu);
        acc.l += p;
        float f[8];
        widen2<DT>(vr[r].x, f[0], f[1]);
        widen2<DT>(vr[r].y, f[2], f[3]);
        widen2<DT>(vr[r].z, f[4], f[5]);
        widen2<DT>(vr[r].w, f[6], f[7]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.o[i] = fmaf(p, f[i], acc.o[i]);
    }
    acc.m = mn;
}

// One step of the streaming loop over the RW rows [kb, kb + RW) of this wave
// (a workgroup step covers CH = 4 RW rows, wave w taking the w-th block).
// K and V are read with different patterns, because they are read side by
// side and their patterns interact: measured with a plain read of 512k's K
// and V on MI355X, K read as 64 bytes of each of 16 rows per instruction next
// to V read as contiguous 1 KiB streams at 7.27 TB/s with all XCDs equally
// fast, where both read contiguously stream at 7.0 TB/s with the odd XCDs
// ~8% slower, and both read as 64-byte pieces at 6.15 TB/s.
//   K: lane (w, c) = (lane / 16, lane % 16) loads 16-byte pieces w + 4 kk
//      (kk < KK) of rows kb + c + 16 sb (sb < SB) and dots them with the same
//      pieces of q; the four lanes w of a row add their parts (two exchanges
//      across 16-lane rows), so every lane ends with the full scores of its
//      rows c + 16 sb.
//   V: lane group g = lane / LPR takes rows kb + GPW i + g (i < kRows), each
//      lane a 16-byte piece `sub` of the row, so one instruction reads GPW
//      whole rows (1 KiB contiguous). The group's scores come from the
//      wave's slice of LDS, where the K lanes leave them.
// Each lane group keeps its own online-softmax state (m, l, Obar of its 8
// dims) over the rows it accumulates. A tail step (the last, partial one)
// clamps rows at or past e to e-1, never reading outside the head, and masks
// their scores to -inf; an edge step (the first one of a range whose step
// grid starts before it, see stream_range) also clamps rows before lo to lo
// and masks them.

template <int DT, int D, int MODE>
__device__ __forceinline__ void stream_step(const char* __restrict__ kh, const char* __restrict__ vh,
                                            int kb, int lo, int e, const uint4 (&qk)[Geo<D>::KK],
                                            float sl2e, float* sx, Acc& acc) {
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int w = lane >> 4, c = lane & 15;
    const int gw = lane / G::LPR, sub = lane % G::LPR;
    uint4 kr[G::SB][G::KK], vr[kRows];
    if constexpr (MODE == kStepFull) {
        const uint32_t koff = (uint32_t)kb * G::RB + (uint32_t)c * G::RB + (uint32_t)w * 16u;
        const uint32_t voff = (uint32_t)kb * G::RB + (uint32_t)lane * 16u;
#pragma unroll
        for (int sb = 0; sb < G::SB; ++sb)
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk)
                kr[sb][kk] = load_nt(kh + (uint64_t)(koff + (uint32_t)sb * 16u * G::RB + kk * 64u));
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            vr[i] = load_nt(vh + (uint64_t)(voff + (uint32_t)i * G::GPW * G::RB));
    } else {
#pragma unroll
        for (int sb = 0; sb < G::SB; ++sb) {
            int r = min(kb + c + 16 * sb, e - 1);
            if constexpr (MODE == kStepEdge) r = max(r, lo);
            const uint32_t j = (uint32_t)r;
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk)
                kr[sb][kk] = load_nt(kh + (uint64_t)(j * G::RB + (uint32_t)(w + 4 * kk) * 16u));
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            int r = min(kb + G::GPW * i + gw, e - 1);
            if constexpr (MODE == kStepEdge) r = max(r, lo);
            const uint32_t j = (uint32_t)r;
            vr[i] = load_nt(vh + (uint64_t)(j * G::RB + (uint32_t)sub * 16u));
        }
    }
    // Keep all the loads of the step in flight before any of them is
    // consumed; without this the scheduler interleaves loads with the math
    // and fewer bytes are outstanding per wave.
    __builtin_amdgcn_sched_barrier(0);
    {
        // The scaled score is rounded once and that same value feeds both the
        // max and exp2(s - m): no contraction of the product into the
        // subtraction, so the maximal row gets weight exactly 1. The four
        // parts of a row are added as (w + w^1) + (w^2 + w^3) in every lane,
        // so all four lanes hold the same bits.
#pragma clang fp contract(off)
#pragma unroll
        for (int sb = 0; sb < G::SB; ++sb) {
            float x = 0.f;
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk) x += dot8<DT>(kr[sb][kk], qk[kk]);
            x = sum_xor16_32(x);
            // row r = c + 16 sb goes to slot (r % GPW) kRows + r / GPW, where
            // group r % GPW finds its rows in order
            const int r = c + 16 * sb;
            if (w == 0) sx[(r % G::GPW) * kRows + r / G::GPW] = x * sl2e;
        }
    }
    __builtin_amdgcn_wave_barrier();
    float s[kRows];
    {
        const float4* src = reinterpret_cast<const float4*>(sx + gw * kRows);
        const float4 s0 = src[0], s1 = src[1];
        s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
        s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    }
    __builtin_amdgcn_wave_barrier();
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int r = kb + G::GPW * i + gw;
        if (MODE != kStepFull && (r >= e || (MODE == kStepEdge && r < lo))) s[i] = kNegInf;
        mx = fmaxf(mx, s[i]);
    }
    const float mn = fmaxf(acc.m, mx);
    const float mu = (mn == kNegInf) ? 0.f : mn;   // no -inf - -inf
    const float alpha = fexp2(acc.m - mu);
    acc.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.o[i] *= alpha;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const float p = fexp2(s[r] - mu);
        acc.l += p;
        float f[8];
        widen2<DT>(vr[r].x, f[0], f[1]);
        widen2<DT>(vr[r].y, f[2], f[3]);
        widen2<DT>(vr[r].z, f[4], f[5]);
        widen2<DT>(vr[r].w, f[6], f[7]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.o[i] = fmaf(p, f[i], acc.o[i]);
    }
    acc.m = mn;
}

// How crowded a workgroup's CU is, for the lean kernel (ctl == nullptr: not
// watched). The 16-row K pattern moves half a cache line per request for K,
// and one CU then reads at most ~34.6 GB/s, against ~48 GB/s for whole-line
// patterns (measured on MI355X with a plain read of each pattern, K and V of
// 4 GiB each, on 128 CUs: 4.43 against 6.18 TB/s). On a whole, uncontended
// device a CU needs ~28 GB/s, so the 16-row blocks win there; when other work
// holds CUs and the launch's workgroups double up on the rest, those CUs need
// more than that ceiling. A wave whose CU holds more than `fair` of the
// launch's workgroups (the per-CU counters of the control block) is crowded
// and reads K by whole rows until it is not. `rows` is this wave's current
// choice.
struct CuWatch {
    const uint32_t* ctl;
    uint32_t slot;
    uint32_t fair;
    bool rows;
};

// A lean peer's flag whose record stores have been issued but not yet waited
// for (wave 0 of a peer whose workgroup has another segment; flag == nullptr
// in every other wave). The wave goes on streaming its next segment and
// raises the flag after that segment's first step: by then the stores have
// had a step's time to complete, so the wait for them that must precede the
// flag store costs the stream nothing.
struct PendingFlag {
    uint32_t* flag;
    uint32_t epoch;
};
__device__ __forceinline__ void raise_pending(PendingFlag* pf) {
    if (pf != nullptr && pf->flag != nullptr) {
        drain_stores();   // the record's stores have completed
        if ((threadIdx.x & 63) == 0)
            __hip_atomic_store(pf->flag, pf->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pf->flag = nullptr;
    }
}

// Stream rows [a, e) of one head (kh/vh point at its row 0, qh at its query
// row) through the lane groups' online softmax; sx is the wave's slice of
// the score exchange in LDS (Geo<D>::RW floats). A head spans less than
// 4 GiB, so every offset inside it fits in 32 bits. A workgroup step covers
// CH rows, wave w its w-th block of RW rows, in either routine.
//
// The two step routines suit different ranges. A long range is bound by the
// rate of its reads, and reads K fastest in 16-row blocks (stream_step); a
// short one is bound by the latency of its few steps, which is lower by
// whole rows with DPP sums (stream_step_rows). Measured on MI355X: 512k
// (ranges of 1024 steps) 1211 us contiguous against 1182 us in 16-row blocks;
// 4096 heads of 2 steps 84 us against 94 us; one uncontended workgroup
// streams 55 GB/s contiguous against 39 GB/s in 16-row blocks. Ranges of at
// least kBlockMinSteps steps take the 16-row blocks, unless `cw` finds the
// CU crowded: every kCheckSteps steps a wave loads its CU's counter with the
// loads of a step and picks the routine of the next steps from it once they
// have arrived, so the look costs no wait.
//
// Long ranges step on a grid that starts at the 4 KiB boundary of the K rows
// at or before row a, so that every 16-row block of K loads covers whole 4 KiB
// blocks: the pattern reads fastest so (measured with a plain read of this
// pattern on MI355X: 7.2-7.3 TB/s aligned, about 3% less at 5-11 rows past a
// boundary), and packed ragged caches put heads at arbitrary rows. The first
// step then masks the rows before a, in either routine.
template <int DT, int D>
__device__ __forceinline__ void stream_range(const uint16_t* kh, const uint16_t* vh, int a, int e,
                                             const uint16_t* qh, float sl2e, float* sx, Acc& acc,
                                             CuWatch* cw = nullptr, PendingFlag* pf = nullptr) {
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const char* kc = reinterpret_cast<const char*>(kh);
    const char* vc = reinterpret_cast<const char*>(vh);
    const uint4 qv = *reinterpret_cast<const uint4*>(qh + (lane % G::LPR) * 8);
    if (e - a < kBlockMinSteps * G::CH) {
        int base = a;
        for (; base + G::CH <= e; base += G::CH) {
            stream_step_rows<DT, D, kStepFull, false>(kc, vc, base, a, e, qv, sl2e, acc);
            raise_pending(pf);
        }
        if (base < e) stream_step_rows<DT, D, kStepTail, false>(kc, vc, base, a, e, qv, sl2e, acc);
        raise_pending(pf);
        return;
    }
    uint4 qk[G::KK];
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk)
        qk[kk] = *reinterpret_cast<const uint4*>(qh + ((lane >> 4) + 4 * kk) * 8);
    const bool watch = cw != nullptr && cw->ctl != nullptr;
    bool rows = watch && cw->rows;
    constexpr uint32_t kAlignRows = 4096 / G::RB;   // 16 at d = 128, 32 at d = 64
    const uint32_t phase = (uint32_t)(((uintptr_t)kc + (uint64_t)(uint32_t)a * G::RB) & 4095u) / G::RB;
    int base = a - (int)min(phase, kAlignRows - 1);
    if (base < a) {
        if (rows)
            stream_step_rows<DT, D, kStepEdge, true>(kc, vc, base + G::RW * wave, a, e, qv, sl2e, acc);
        else
            stream_step<DT, D, kStepEdge>(kc, vc, base + G::RW * wave, a, e, qk, sl2e, sx, acc);
        base += G::CH;
        raise_pending(pf);
    }
    for (int j = 1; base + G::CH <= e; base += G::CH, ++j) {
        const bool look = watch && (j % kCheckSteps) == 0;
        uint32_t count = 0;
        if (look) count = cu_count(cw->ctl, cw->slot);   // arrives with the step's loads
        if (rows)
            stream_step_rows<DT, D, kStepFull, true>(kc, vc, base + G::RW * wave, a, e, qv, sl2e, acc);
        else
            stream_step<DT, D, kStepFull>(kc, vc, base + G::RW * wave, a, e, qk, sl2e, sx, acc);
        if (look) rows = __builtin_amdgcn_readfirstlane(count) > cw->fair;
        raise_pending(pf);
    }
    if (base < e) {
        if (rows)
            stream_step_rows<DT, D, kStepTail, true>(kc, vc, base + G::RW * wave, a, e, qv, sl2e, acc);
        else
            stream_step<DT, D, kStepTail>(kc, vc, base + G::RW * wave, a, e, qk, sl2e, sx, acc);
    }
    raise_pending(pf);
    if (watch) cw->rows = rows;
}

// NS sets of fold state. The lean kernel keeps two, used by alternate
// segments: its waves 1-3 leave a fold without waiting for wave 0 to read it,
// since the next fold writes the other set, and the one after that waits at
// its barrier for wave 0, which has finished reading by then.
template <int D, int NS = 1>
struct alignas(16) Smem {
    float o[NS][Geo<D>::NG][D];
    float m[NS][Geo<D>::NG];
    float l[NS][Geo<D>::NG];
    float sx[kWaves][Geo<D>::RW];   // per wave: the scores of its step, for its V lanes
};

// Dims of the output each lane of wave 0 holds after a fold: lane i holds
// dims i, i + 64, ... (coalesced 256-byte rows per k).
template <int D>
constexpr int kDpl = D / 64;

// Fold the lane groups of the workgroup with f, through fold state set
// `set` (0 or 1). Wave 0 receives (m, l, Obar[lane + 64k]) of everything the
// workgroup streamed for this range. With kTrail the other waves return after
// a second barrier, once wave 0 has read the state; without it they return at
// once, and the caller's next fold must use the other set.
template <int D, bool kTrail = true, int NS>
__device__ __forceinline__ void wg_fold(Smem<D, NS>& sm, int set, const Acc& a, int grp, int sub,
                                        float& M, float& Ls, float (&O)[kDpl<D>]) {
    using G = Geo<D>;
    float4* dst = reinterpret_cast<float4*>(&sm.o[set][grp][sub * 8]);
    dst[0] = make_float4(a.o[0], a.o[1], a.o[2], a.o[3]);
    dst[1] = make_float4(a.o[4], a.o[5], a.o[6], a.o[7]);
    if (sub == 0) {
        sm.m[set][grp] = a.m;
        sm.l[set][grp] = a.l;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 64) {
        float mx = kNegInf;
#pragma unroll
        for (int g = 0; g < G::NG; ++g) mx = fmaxf(mx, sm.m[set][g]);
        const float mu = (mx == kNegInf) ? 0.f : mx;
        float ls = 0.f, o[kDpl<D>];
#pragma unroll
        for (int k = 0; k < kDpl<D>; ++k) o[k] = 0.f;
#pragma unroll 8
        for (int g = 0; g < G::NG; ++g) {
            const float w = fexp2(sm.m[set][g] - mu);
            ls = fmaf(w, sm.l[set][g], ls);
#pragma unroll
            for (int k = 0; k < kDpl<D>; ++k) o[k] = fmaf(w, sm.o[set][g][t + 64 * k], o[k]);
        }
        M = mx;
        Ls = ls;
#pragma unroll
        for (int k = 0; k < kDpl<D>; ++k) O[k] = o[k];
    }
    if constexpr (kTrail) __syncthreads();
}


// Wave 0 writes out = Obar / l (and m in natural-log units, l) for head u.
template <int D>
__device__ __forceinline__ void write_out(float* out, float* m_out, float* l_out, int u, int lane,
                                          float M, float Ls, const float (&O)[kDpl<D>]) {
    const float inv = 1.f / Ls;
#pragma unroll
    for (int k = 0; k < kDpl<D>; ++k) out[(int64_t)u * D + lane + 64 * k] = O[k] * inv;
    if (lane == 0) {
        if (m_out != nullptr) m_out[u] = M * kLn2;
        if (l_out != nullptr) l_out[u] = Ls;
    }
}

// ------------------------------------------------------------------ lean

template <int DT, int D, int SRC>
__global__ __launch_bounds__(kThreads) void lean_kernel(const LeanArgs a) {
    using G = Geo<D>;
    constexpr int P = kDpl<D>;
    __shared__ Smem<D, 2> sm;
    const int c = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int grp = (t >> 6) * G::GPW + lane / G::LPR;
    const int sub = lane % G::LPR;
    const uint64_t t_in = stamp_start(a.ts, c);
    const uint32_t ep = launch_epoch(a.ctl);
    __shared__ SchedLds sl;
    SegCursor<SRC> cur(a.sched, kernarg_sched<LeanArgs>(), sl, c);
    if (cur.bad()) {   // lengths from device memory out of range: nothing is computed
        if (c == 0 && t == 0) atomicOr(&a.ctl[kCtlErr], kErrLengths);
        if (t == 0) launch_exit(a.ctl, ep);
        stamp_end(a.ts, c);
        return;
    }
    CuWatch cw{a.cu_fair > 0 ? a.ctl : nullptr, cu_slot(), (uint32_t)a.cu_fair, false};
    if (cw.ctl != nullptr && t == 0) cu_add(a.ctl, cw.slot, 1);
    LeanSeg sg;
    int set = 0;             // fold state set of the next segment (alternates)
    PendingFlag pf{nullptr, 0u};
    while (cur.next(sg)) {
        const int u = sg.u;
        const int n = sg.n;
        const int64_t row0 = head_row0(a.kv_stride, a.H, sg.b, sg.unit, sg.tok_off, n);
        const int tok0 = sg.t0 * a.L;
        const int tok1 = (int)min((int64_t)sg.t1 * a.L, (int64_t)n);
        Acc acc;
        acc_init(acc);
        {
            // With uniform contexts every workgroup's range starts at the same
            // offset in its head, and the workgroups, streaming at one rate,
            // read the same address phase at the same time. A long range then
            // starts at one of eight per-workgroup steps, wraps around and
            // ends where it would have started; the order of the tiles does
            // not change the result beyond rounding. Measured on MI355X, old
            // and new library interleaved in one process: 1-2.6% faster on
            // d = 64 heads of 64k tokens (56 heads on 1, 2 and 4 requests, 192
            // heads), 0.9% on 65k and 1% on 512k-h4, 512k unchanged; on the
            // ragged batch, whose packed heads already start at scattered
            // phases, the same rotation cost 0.8%, so it is used only for
            // uniform lengths (seen by the host, or by the launch itself when
            // it reads them from device memory).
            using GG = Geo<D>;
            const int nsteps = (tok1 - tok0) / GG::CH;
            const bool uniform = a.rotate != 0 || cur.uniform();
            const int rot = uniform && nsteps >= 4 * kBlockMinSteps ? ((c * 5) & 7) * (nsteps >> 3) : 0;
            const int mid = tok0 + rot * GG::CH;
            if (rot > 0) {
                stream_range<DT, D>(a.k + row0 * D, a.v + row0 * D, mid, tok1, a.q + (int64_t)u * D,
                                    a.sl2e, sm.sx[t >> 6], acc, &cw, &pf);
                stream_range<DT, D>(a.k + row0 * D, a.v + row0 * D, tok0, mid, a.q + (int64_t)u * D,
                                    a.sl2e, sm.sx[t >> 6], acc, &cw, &pf);
            } else {
                stream_range<DT, D>(a.k + row0 * D, a.v + row0 * D, tok0, tok1, a.q + (int64_t)u * D,
                                    a.sl2e, sm.sx[t >> 6], acc, &cw, &pf);
            }
        }
        if (a.tile_owner != nullptr && t == 0)
            for (int i = sg.t0; i < sg.t1; ++i) a.tile_owner[sg.iter0 + i - sg.t0] = c;

        float M = kNegInf, Ls = 0.f, O[P];
#pragma unroll
        for (int k = 0; k < P; ++k) O[k] = 0.f;   // waves 1-3 start a wide merge from zero
        // Waves 1-3 leave the fold without waiting for wave 0 to read it and
        // go on to the next segment, whose fold uses the other state set.
        wg_fold<D, false>(sm, set, acc, grp, sub, M, Ls, O);
        set ^= 1;
        // A host's segment is the last of its workgroup's range. With more
        // than kMergeBatch peers, all four waves wait for and fold a quarter
        // of them each; otherwise the epilogue is wave 0's and the others go
        // on streaming.
        const bool wide = sg.host && !sg.fin && sg.last - c > kMergeBatch;
        if (t >= 64 && !wide) continue;

        if (!sg.host) {
            // a peer: publish (Obar, m, l) for the head's host; the flag goes
            // up to this launch's epoch once the stores have completed -- after
            // the first step of the workgroup's next segment, or at its end
            float* p = a.part + (int64_t)c * part_stride(D);
#pragma unroll
            for (int k = 0; k < P; ++k) store_agent(p + lane + 64 * k, O[k]);
            if (lane == 0) {
                store_agent(p + D, M);
                store_agent(p + D + 1, Ls);
            }
            pf = PendingFlag{&a.flags[c], ep};
            continue;
        }
        if (!sg.fin) {
            // The host. Its peers (c, last] each publish one partial: wait for
            // all of them at once (one flag per lane), then fold them in
            // ascending workgroup order with their loads issued in batches.
            // With many peers, wave w takes the w-th quarter of them (wave 0
            // on top of the host's own state) and wave 0 then folds the other
            // waves' states in wave order: a fixed order, so the bits do not
            // depend on timing.
            const int wave = t >> 6;
            const int np = sg.last - c;
            const int q = wide ? (np + kWaves - 1) / kWaves : np;
            const int p_first = c + 1 + wave * q;
            const int p_last = min(p_first + q - 1, sg.last);
            const uint64_t w0 = stamp_now(a.ts);
            for (int i = lane; i <= p_last - p_first; i += 64)
                wait_flag(&a.flags[p_first + i], ep, a.wait_ticks, a.ctl);
            if (wave == 0) stamp_wait(a.ts, c, t_in, w0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            for (int p0 = p_first; p0 <= p_last; p0 += kMergeBatch) {
                float pm[kMergeBatch], pl[kMergeBatch], po[kMergeBatch][P];
#pragma unroll
                for (int j = 0; j < kMergeBatch; ++j) {
                    const float* p = a.part + (int64_t)min(p0 + j, p_last) * part_stride(D);
                    pm[j] = load_agent(p + D);
                    pl[j] = load_agent(p + D + 1);
#pragma unroll
                    for (int k = 0; k < P; ++k) po[j][k] = load_agent(p + lane + 64 * k);
                }
#pragma unroll
                for (int j = 0; j < kMergeBatch; ++j)
                    if (p0 + j <= p_last) merge_into<P>(M, Ls, O, pm[j], pl[j], po[j]);
            }
            if (wide) {
                // through the state set the fold did not use: wave 0 read
                // that one before the fold's barrier
                if (wave > 0) {
#pragma unroll
                    for (int k = 0; k < P; ++k) sm.o[set][wave][lane + 64 * k] = O[k];
                    if (lane == 0) {
                        sm.m[set][wave] = M;
                        sm.l[set][wave] = Ls;
                    }
                }
                __syncthreads();
                if (wave > 0) continue;
                for (int v = 1; v < kWaves; ++v) {
                    float ov[P];
#pragma unroll
                    for (int k = 0; k < P; ++k) ov[k] = sm.o[set][v][lane + 64 * k];
                    merge_into<P>(M, Ls, O, sm.m[set][v], sm.l[set][v], ov);
                }
            }
        }
        write_out<D>(a.out, a.m_out, a.l_out, u, lane, M, Ls, O);
    }
    raise_pending(&pf);   // a peer segment that was its workgroup's last
    if (cw.ctl != nullptr && t == 0) cu_add(a.ctl, cw.slot, -1);
    if (t == 0) launch_exit(a.ctl, ep);
    stamp_end(a.ts, c);
}

// ------------------------------------------------------------------ dynamic pull

// Record slot of a head's piece in chunk ch: (ch, 0) if the piece starts the
// chunk, else (ch, 1) -- the chunk's last, partial segment.
__device__ __forceinline__ int piece_slot(int ch, int Su, int C) {
    return ch * 2 + (max(Su, ch * C) == ch * C ? 0 : 1);
}

// Wave 0 stores a record (Obar, m, l) with device-coherent stores.
template <int D>
__device__ __forceinline__ void publish_rec(float* p, int lane, float M, float Ls,
                                            const float (&O)[kDpl<D>]) {
#pragma unroll
    for (int j = 0; j < kDpl<D>; ++j) store_agent(p + lane + 64 * j, O[j]);
    if (lane == 0) {
        store_agent(p + D, M);
        store_agent(p + D + 1, Ls);
    }
}

// After this wave's records are stored: wait for them to complete, then add
// one to the counter. True for the wave whose add brings it to `last` + 1
// (the last arrival), which then owns the merge.
__device__ __forceinline__ bool count_in(uint32_t* ctr, uint32_t last, int lane) {
    drain_stores();
    uint32_t before = 0;
    if (lane == 0)
        before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    before = __shfl(before, 0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return before == last;
}

// Wave 0 folds, in order, the records of chunks ch0, ch0 + step, ... (n of
// them) of one head from `base` into (M, Ls, O), replacing what they held.
template <int D>
__device__ __forceinline__ void fold_slots(const float* base, int ch0, int n, int step, int Su,
                                           int C, int lane, float& M, float& Ls,
                                           float (&O)[kDpl<D>]) {
    constexpr int P = kDpl<D>;
    constexpr int kBatch = 16;
    M = kNegInf;
    Ls = 0.f;
#pragma unroll
    for (int j = 0; j < P; ++j) O[j] = 0.f;
    for (int i0 = 0; i0 < n; i0 += kBatch) {
        float pm[kBatch], pl[kBatch], po[kBatch][P];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int ch = ch0 + min(i0 + j, n - 1) * step;
            const float* rp = base + (int64_t)piece_slot(ch, Su, C) * part_stride(D);
            pm[j] = load_agent(rp + D);
            pl[j] = load_agent(rp + D + 1);
#pragma unroll
            for (int x = 0; x < P; ++x) po[j][x] = load_agent(rp + lane + 64 * x);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (i0 + j < n) merge_into<P>(M, Ls, O, pm[j], pl[j], po[j]);
    }
}

// Stream-K over fixed chunks of the tile sequence, taken dynamically (the
// digest's CTAs that pull the next tile instead of holding a fixed split) or
// one per workgroup (a non-persistent grid). Pieces of a head that spans
// several chunks are merged by whichever workgroup finishes the last of them,
// in chunk order, so the result does not depend on which workgroup took which
// chunk. No workgroup waits for another: any grid size is safe.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void pull_kernel(const PullArgs a) {
    using G = Geo<D>;
    constexpr int P = kDpl<D>;
    __shared__ Smem<D> sm;
    __shared__ int s_chunk;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int grp = (t >> 6) * G::GPW + lane / G::LPR;
    const int sub = lane % G::LPR;
    stamp_start(a.ts, blockIdx.x);
    CuWatch cw{a.cu_fair > 0 ? a.ctl : nullptr, cu_slot(), (uint32_t)a.cu_fair, false};
    if (cw.ctl != nullptr && t == 0) cu_add(a.ctl, cw.slot, 1);
    // A workgroup takes its next chunk only when it has finished the last one
    // (taking it earlier hands chunks to workgroups that are still busy while
    // others, started later, find none).
    int next = blockIdx.x;
    if (a.dynamic) {
        if (t == 0)
            s_chunk = (int)__hip_atomic_fetch_add(&a.pull[0], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        next = s_chunk;
        __syncthreads();
    }
    for (;;) {
        const int k = next;
        if (k >= a.nchunks) break;
        const int c0 = k * a.C;
        const int c1 = min(c0 + a.C, a.I);
        int u = a.chunk_head[k];
        for (int it = c0; it < c1; ++u) {
            const int Su = a.head_start[u], Se = a.head_start[u + 1];
            const int t1 = min(Se, c1);
            const int b = u / a.H;
            const int h = u - b * a.H;
            const int n = a.ctx[b];
            const int64_t row0 = head_row0(a.kv_stride, a.H, b, h, a.tok_off[b], n);
            const int tok0 = (it - Su) * a.L;
            const int tok1 = (int)min((int64_t)(t1 - Su) * a.L, (int64_t)n);
            Acc acc;
            acc_init(acc);
            stream_range<DT, D>(a.k + row0 * D, a.v + row0 * D, tok0, tok1,
                                a.q + (int64_t)u * D, a.sl2e, sm.sx[t >> 6], acc, &cw);
            if (a.tile_owner != nullptr)
                for (int i = it + t; i < t1; i += kThreads) a.tile_owner[i] = blockIdx.x;
            float M = kNegInf, Ls = 0.f, O[P];
            wg_fold<D>(sm, 0, acc, grp, sub, M, Ls, O);
            const int side = it == c0 ? 0 : 1;
            it = t1;
            if (t >= 64) continue;   // the epilogue is wave 0's

            const int kf = Su / a.C, kl = (Se - 1) / a.C;   // chunks holding head u
            if (kf != kl) {
                // A piece of a head spread over chunks kf..kl. Level 1: the
                // chunks form groups of kMergeFanIn; the last piece of a group
                // to arrive folds the group's pieces in chunk order. Level 2:
                // the last group folds the group results in order. The tree is
                // fixed, so the bits do not depend on who arrives last.
                const int g0 = kf + (k - kf) / kMergeFanIn * kMergeFanIn;
                const int g1 = min(g0 + kMergeFanIn - 1, kl);
                const int ngroups = (kl - kf) / kMergeFanIn + 1;
                const int gslot = piece_slot(g0, Su, a.C);
                if (g1 > g0) {
                    publish_rec<D>(a.part + (int64_t)(k * 2 + side) * part_stride(D), lane, M, Ls, O);
                    if (!count_in(&a.gcount[gslot], (uint32_t)(g1 - g0), lane)) continue;
                    fold_slots<D>(a.part, g0, g1 - g0 + 1, 1, Su, a.C, lane, M, Ls, O);
                    if (lane == 0)
                        __hip_atomic_store(&a.gcount[gslot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (ngroups > 1) {
                    float* l1 = a.part + (int64_t)2 * a.nchunks * part_stride(D);
                    publish_rec<D>(l1 + (int64_t)gslot * part_stride(D), lane, M, Ls, O);
                    if (!count_in(&a.arrive[u], (uint32_t)(ngroups - 1), lane)) continue;
                    fold_slots<D>(l1, kf, ngroups, kMergeFanIn, Su, a.C, lane, M, Ls, O);
                    if (lane == 0)
                        __hip_atomic_store(&a.arrive[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            write_out<D>(a.out, a.m_out, a.l_out, u, lane, M, Ls, O);
        }
        if (a.dynamic) {
            __syncthreads();
            if (t == 0)
                s_chunk = (int)__hip_atomic_fetch_add(&a.pull[0], 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            next = s_chunk;
        } else {
            next = a.nchunks;
        }
    }
    if (cw.ctl != nullptr && t == 0) cu_add(a.ctl, cw.slot, -1);
    if (a.dynamic && t == 0) {
        // the last workgroup out re-arms the counters for the next launch
        const uint32_t done = __hip_atomic_fetch_add(&a.pull[1], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&a.pull[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.pull[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    stamp_end(a.ts, blockIdx.x);
}

// ------------------------------------------------------------------ fixed split

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void split_kernel(const SplitArgs a) {
    using G = Geo<D>;
    constexpr int P = kDpl<D>;
    __shared__ Smem<D> sm;
    stamp_start(a.ts, blockIdx.x);
    const int u = blockIdx.x / a.splits;
    const int k = blockIdx.x - u * a.splits;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int grp = (t >> 6) * G::GPW + lane / G::LPR;
    const int sub = lane % G::LPR;
    const int b = u / a.H;
    const int h = u - b * a.H;
    const int n = a.ctx[b];
    const int64_t row0 = head_row0(a.kv_stride, a.H, b, h, a.tok_off[b], n);
    const int64_t T = ((int64_t)n + a.L - 1) / a.L;
    const int64_t t0 = (int64_t)k * T / a.splits, t1 = (int64_t)(k + 1) * T / a.splits;
    const int tok0 = (int)(t0 * a.L);
    const int tok1 = (int)min(t1 * a.L, (int64_t)n);
    Acc acc;
    acc_init(acc);
    if (tok0 < tok1)
        stream_range<DT, D>(a.k + row0 * D, a.v + row0 * D, tok0, tok1, a.q + (int64_t)u * D,
                            a.sl2e, sm.sx[t >> 6], acc);
    float M = kNegInf, Ls = 0.f, O[P];
    wg_fold<D>(sm, 0, acc, grp, sub, M, Ls, O);
    if (t >= 64) return;
    float* p = a.part + (int64_t)blockIdx.x * part_stride(D);
#pragma unroll
    for (int j = 0; j < P; ++j) p[lane + 64 * j] = O[j];
    if (lane == 0) {
        p[D] = M;
        p[D + 1] = Ls;
    }
    stamp_end(a.ts, blockIdx.x);
}

// One wave per head: folds the head's `splits` partial records in order.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const CombineArgs a) {
    constexpr int P = kDpl<D>;
    const int u = blockIdx.x;
    const int lane = threadIdx.x;
    float M = kNegInf, Ls = 0.f, O[P];
#pragma unroll
    for (int j = 0; j < P; ++j) O[j] = 0.f;
    for (int k = 0; k < a.splits; ++k) {
        const float* p = a.part + ((int64_t)u * a.splits + k) * part_stride(D);
        float po[P];
#pragma unroll
        for (int j = 0; j < P; ++j) po[j] = p[lane + 64 * j];
        merge_into<P>(M, Ls, O, p[D], p[D + 1], po);
    }
    write_out<D>(a.out, a.m_out, a.l_out, u, lane, M, Ls, O);
}

// ------------------------------------------------------------------ per head

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void per_head_kernel(const SplitArgs a) {
    using G = Geo<D>;
    __shared__ Smem<D> sm;
    stamp_start(a.ts, blockIdx.x);
    const int u = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int grp = (t >> 6) * G::GPW + lane / G::LPR;
    const int sub = lane % G::LPR;
    const int b = u / a.H;
    const int h = u - b * a.H;
    const int n = a.ctx[b];
    const int64_t row0 = head_row0(a.kv_stride, a.H, b, h, a.tok_off[b], n);
    Acc acc;
    acc_init(acc);
    stream_range<DT, D>(a.k + row0 * D, a.v + row0 * D, 0, n, a.q + (int64_t)u * D, a.sl2e,
                        sm.sx[t >> 6], acc);
    float M = kNegInf, Ls = 0.f, O[kDpl<D>];
    wg_fold<D>(sm, 0, acc, grp, sub, M, Ls, O);
    if (t < 64) write_out<D>(a.out, a.m_out, a.l_out, u, lane, M, Ls, O);
    stamp_end(a.ts, blockIdx.x);
}

// The achievable streaming-read bandwidth of the device, for measurement: the
// loads of the attention kernels without their arithmetic. Each workgroup
// reads one contiguous chunk as two halves side by side, a "K" half and a
// "V" half, in trips of 32 KiB per half (8 KiB per wave): K as 64 bytes of
// each of 16 rows of 256 bytes per instruction, V as contiguous 1 KiB per
// instruction, 16 non-temporal 16-byte loads per lane in flight -- the load
// pattern of a d = 128 streaming step. The data are folded into one word so
// the loads stay; the word is stored only in the (practically impossible)
// case that it equals a fixed pattern.
constexpr int kReadTrip = 64 << 10;   // bytes per workgroup trip, both halves
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, uint64_t chunk,
                                                                uint32_t* sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int w = lane >> 4, c = lane & 15;
    const uint64_t half = chunk / 2;
    const char* kb = src + blockIdx.x * chunk + (uint64_t)wave * 8192u;
    const char* vb = kb + half;
    const uint32_t koff = (uint32_t)c * 256u + (uint32_t)w * 16u;
    const uint32_t voff = (uint32_t)lane * 16u;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (uint64_t off = 0; off < half; off += kReadTrip / 2) {
        u32x4_t v[16];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                v[4 * sb + kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                    kb + off + koff + (uint32_t)sb * 4096u + (uint32_t)kk * 64u));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[8 + i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(vb + off + voff + (uint32_t)i * 1024u));
        __builtin_amdgcn_sched_barrier(0);   // all loads of the trip in flight first
#pragma unroll
        for (int k = 0; k < 16; ++k) acc ^= v[k];
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

template <typename F>
const void* pick(int dtype, int d, F f16_64, F f16_128, F bf16_64, F bf16_128) {
    if (dtype == 0) return d == 64 ? (const void*)f16_64 : (const void*)f16_128;
    return d == 64 ? (const void*)bf16_64 : (const void*)bf16_128;
}

}  // namespace

const void* lean_kernel_ptr(int dtype, int d, int src) {
    if (src == kSrcArgs)
        return pick(dtype, d, &lean_kernel<0, 64, kSrcArgs>, &lean_kernel<0, 128, kSrcArgs>,
                    &lean_kernel<1, 64, kSrcArgs>, &lean_kernel<1, 128, kSrcArgs>);
    if (src == kSrcDevice)
        return pick(dtype, d, &lean_kernel<0, 64, kSrcDevice>, &lean_kernel<0, 128, kSrcDevice>,
                    &lean_kernel<1, 64, kSrcDevice>, &lean_kernel<1, 128, kSrcDevice>);
    return pick(dtype, d, &lean_kernel<0, 64, kSrcTables>, &lean_kernel<0, 128, kSrcTables>,
                &lean_kernel<1, 64, kSrcTables>, &lean_kernel<1, 128, kSrcTables>);
}

hipError_t launch_lean(int dtype, int d, const LeanArgs& a, int grid, hipStream_t s,
                       bool cooperative) {
    const void* fn = lean_kernel_ptr(dtype, d, a.sched.src);
    void* args[] = {const_cast<LeanArgs*>(&a)};
    if (cooperative)
        return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

uint64_t stream_read_unit() { return (uint64_t)kReadTrip; }

hipError_t launch_stream_read(const void* src, uint64_t chunk, int grid, uint32_t* sink,
                              hipStream_t s) {
    const char* p = static_cast<const char*>(src);
    void* args[] = {&p, &chunk, &sink};
    return hipLaunchKernel((const void*)&stream_read_kernel, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_pull(int dtype, int d, const PullArgs& a, int grid, hipStream_t s) {
    const void* fn = pick(dtype, d, &pull_kernel<0, 64>, &pull_kernel<0, 128>, &pull_kernel<1, 64>,
                          &pull_kernel<1, 128>);
    void* args[] = {const_cast<PullArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_split(int dtype, int d, const SplitArgs& a, int blocks, hipStream_t s) {
    const void* fn = pick(dtype, d, &split_kernel<0, 64>, &split_kernel<0, 128>,
                          &split_kernel<1, 64>, &split_kernel<1, 128>);
    void* args[] = {const_cast<SplitArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(blocks), dim3(kThreads), args, 0, s);
}

hipError_t launch_combine(int d, const CombineArgs& a, int heads, hipStream_t s) {
    const void* fn = d == 64 ? (const void*)&combine_kernel<64> : (const void*)&combine_kernel<128>;
    void* args[] = {const_cast<CombineArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(heads), dim3(64), args, 0, s);
}

hipError_t launch_per_head(int dtype, int d, const SplitArgs& a, int heads, hipStream_t s) {
    const void* fn = pick(dtype, d, &per_head_kernel<0, 64>, &per_head_kernel<0, 128>,
                          &per_head_kernel<1, 64>, &per_head_kernel<1, 128>);
    void* args[] = {const_cast<SplitArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(heads), dim3(kThreads), args, 0, s);
}

}  // namespace la
