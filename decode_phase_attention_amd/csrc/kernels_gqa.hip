// Grouped-query decode attention on gfx950: g = H / Hk query heads share one
// K/V head, so every K/V row meets up to 16 query rows at once and the scores
// and the weighted sum form dense tiles. Both go through the 16x16x32 MFMA:
//
//   S^T (keys x q)  = K (keys x d)  . Q^T (d x q)        k-dim: head dim
//   O^T (d x q)    += V^T (d x keys) . P^T (keys x q)    k-dim: keys
//
// Operand layout of v_mfma_f32_16x16x32_{bf16,f16} (lane l, w = l/16,
// c = l%16): A[c][8w + j], B[8w + j][c], C[4w + r][c]. Two freedoms make every
// operand a direct 16-byte load from HBM (no LDS staging):
//   - the order of a contraction is free, so lane (w, c) loads K row c at
//     16-byte piece w + 4kk and Q row c at the same piece;
//   - the d index of a row of O^T is free, so O^T row i of block nb is head
//     dim NB*i + nb: lane (w, c) then needs V[key][NB*c .. NB*c + NB) -- one
//     contiguous load per key -- and an in-register 8 x NB transpose (v_perm)
//     turns its 8 keys x NB dims into the A operands of the NB blocks.
// The S^T accumulator leaves lane (w, c) holding query c's scores for keys
// 4w + r + 16sb, exactly the 8 keys it loaded V for, so P^T needs no shuffle.
// P is split into a 16-bit high and low part (two MFMAs) so that the weighted
// sum keeps ~16 significant bits of every weight instead of 8.
//
// The query columns of a K/V head are its g query heads times the Nq new
// tokens of the request, ordered (head in group, token). Token t of Nq sits
// at cache position n - Nq + t and sees keys [0, n - Nq + t], so keys below
// n - Nq + 1 are seen by every column and only the last steps of a head mask
// per column. Columns beyond the g * Nq live ones are zero and never
// written. More than 16 columns are cut into blocks of 16, each a unit of the
// schedule (the K/V head is then streamed once per block).
//
// Each wave streams 32 keys per step with its own online softmax (per query
// column: m, a per-lane partial l, O^T); waves meet in LDS only at the end of
// a range. A lean segment steps on a grid that starts at the 4 KiB boundary
// of its K rows (see gseg_start). The epilogue uses all 256 threads: thread t owns query t / 16 and
// head dims [(t % 16) * D/16, +D/16), so a wave covers four whole records.
// The exchange between workgroups is the same agent-scope, completion-ordered
// protocol as the single-head kernels, with 16 records (one per query column)
// per workgroup, moved in 16-byte device-coherent buffer accesses. The same
// four decompositions exist as for single heads: lean (static stream-K),
// pull (chunks taken from a counter, merged by the last piece), fixed split +
// combine, and per unit.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace la {

namespace {

static_assert(kThreads == 256, "the grouped epilogue maps 16 queries x 16 dim chunks to 256 threads");

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct GGeo {
    static constexpr int RB = D * 2;            // bytes per K/V row
    static constexpr int KK = D / 32;           // MFMA k-chunks of the head dim: 4 or 2
    static constexpr int NB = D / 16;           // 16-row blocks of O^T: 8 or 4
    static constexpr int KEYS = 32;             // keys per wave step
    static constexpr int CH = KEYS * kWaves;    // keys per workgroup step: 128
    static constexpr int DPT = D / 16;          // epilogue dims per thread: 8 or 4
    static constexpr int VW = NB / 2;           // 32-bit words of V per lane per key: 4 or 2
};

template <int DT>
__device__ __forceinline__ f32x4_t mfma(const u32x4_t a, const u32x4_t b, const f32x4_t c) {
    if constexpr (DT == 0)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Round p to the 16-bit input type, and the remainder too: hi + lo carries
// ~16 significant bits of p into the MFMA.
template <int DT>
__device__ __forceinline__ void split_p(const float (&p)[8], u32x4_t& hi, u32x4_t& lo) {
    if constexpr (DT == 0) {
        f16x8_t h, l;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h[j] = (_Float16)p[j];
            l[j] = (_Float16)(p[j] - (float)h[j]);
        }
        hi = __builtin_bit_cast(u32x4_t, h);
        lo = __builtin_bit_cast(u32x4_t, l);
    } else {
        bf16x8_t h, l;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h[j] = (__bf16)p[j];
            l[j] = (__bf16)(p[j] - (float)h[j]);
        }
        hi = __builtin_bit_cast(u32x4_t, h);
        lo = __builtin_bit_cast(u32x4_t, l);
    }
}

__device__ __forceinline__ u32x4_t load16(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

template <int D>
struct GState {
    float m;                        // running max of query c, log2 units
    float l;                        // this lane's partial sum of 2^(s - m)
    f32x4_t o[GGeo<D>::NB];         // O^T blocks: o[nb][r] = O[c][NB*(4w + r) + nb]
};

template <int D>
__device__ __forceinline__ void gstate_init(GState<D>& st) {
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int nb = 0; nb < GGeo<D>::NB; ++nb) st.o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// K/V registers of one wave step (32 keys).
template <int D>
struct GRegs {
    u32x4_t kr[2][GGeo<D>::KK];         // lane (w, c): key c (+16 sb), 16-byte piece w + 4kk
    uint32_t vr[8][GGeo<D>::VW];        // keys 4w + r + 16sb (j = r + 4sb), dims [NB*c, NB*c + NB)
};

// Kinds of wave step: every key valid; keys from a lane's limit masked (the
// last steps of a range); and keys before the range start masked too (the
// first step of a range whose step grid starts before it, see gseg_start).
constexpr int kStepFull = 0, kStepTail = 1, kStepEdge = 2;
constexpr int kAlignMinSteps = 4;

// Issue the loads of one wave step over keys [kb, kb + 32) of a head (rows of
// kh/vh). A tail step keeps loads below e; an edge step keeps them in [lo, e).
template <int D, int MODE>
__device__ __forceinline__ void gqa_load(const char* __restrict__ kh, const char* __restrict__ vh,
                                         int kb, int lo, int e, int w, int c, GRegs<D>& g) {
    using G = GGeo<D>;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        int key = kb + c + 16 * sb;
        if constexpr (MODE == kStepTail) key = min(key, e - 1);
        if constexpr (MODE == kStepEdge) key = min(max(key, lo), e - 1);
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk)
            g.kr[sb][kk] = load16(kh + (uint64_t)((uint32_t)key * G::RB + (uint32_t)(w + 4 * kk) * 16u));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int key = kb + 4 * w + (j & 3) + 16 * (j >> 2);
        if constexpr (MODE == kStepTail) key = min(key, e - 1);
        if constexpr (MODE == kStepEdge) key = min(max(key, lo), e - 1);
        const char* src = vh + (uint64_t)((uint32_t)key * G::RB + (uint32_t)c * (G::NB * 2));
        if constexpr (G::VW == 4) {
            const u32x4_t x = load16(src);
            g.vr[j][0] = x.x; g.vr[j][1] = x.y; g.vr[j][2] = x.z; g.vr[j][3] = x.w;
        } else {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(src));
            g.vr[j][0] = x.x; g.vr[j][1] = x.y;
        }
    }
}

// The arithmetic of one wave step on loaded registers. In a tail step this
// lane's query column masks keys >= lim; an edge step also masks keys < lo.
// qt[kk] is the B operand of Q^T for head-dim chunk kk.
template <int DT, int D, int MODE>
__device__ __forceinline__ void gqa_compute(const GRegs<D>& g, int kb, int lo, int lim, int w,
                                            const u32x4_t (&qt)[GGeo<D>::KK], float sl2e,
                                            GState<D>& st) {
    using G = GGeo<D>;
    // scores S^T: lane holds s[j] = S[q = c][key = kb + 4w + (j & 3) + 16 (j >> 2)]
    float s[8];
    {
#pragma clang fp contract(off)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk) acc = mfma<DT>(g.kr[sb][kk], qt[kk], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = acc[r] * sl2e;
                const int key = kb + 4 * w + r + 16 * sb;
                const bool ok = MODE == kStepFull ? true
                              : MODE == kStepTail ? key < lim
                                                  : (key >= lo && key < lim);
                s[r + 4 * sb] = ok ? x : kNegInf;
            }
        }
    }
    // online softmax of query c across the 4 lanes (w = 0..3) that hold its keys
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, s[j]);
    mx = max_xor16_32(mx);
    const float mn = fmaxf(st.m, mx);
    const float mu = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fexp2(st.m - mu);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = fexp2(s[j] - mu);
        ps += p[j];
    }
    st.l = st.l * alpha + ps;
    st.m = mn;
    u32x4_t phi, plo;
    split_p<DT>(p, phi, plo);
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
        // A operand of block nb: V[key(j)][NB*c + nb] for j = 0..7 (8 x NB transpose)
        const int wd = nb >> 1;
        const uint32_t sel = (nb & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t a;
        a.x = __builtin_amdgcn_perm(g.vr[1][wd], g.vr[0][wd], sel);
        a.y = __builtin_amdgcn_perm(g.vr[3][wd], g.vr[2][wd], sel);
        a.z = __builtin_amdgcn_perm(g.vr[5][wd], g.vr[4][wd], sel);
        a.w = __builtin_amdgcn_perm(g.vr[7][wd], g.vr[6][wd], sel);
        f32x4_t o = st.o[nb] * alpha;
        o = mfma<DT>(a, phi, o);
        o = mfma<DT>(a, plo, o);
        st.o[nb] = o;
    }
}

// One wave step over keys [kb, kb + 32): all loads in flight, then the
// arithmetic.
template <int DT, int D, bool TAIL>
__device__ __forceinline__ void gqa_step(const char* __restrict__ kh, const char* __restrict__ vh,
                                         int kb, int e, int lim, int w, int c,
                                         const u32x4_t (&qt)[GGeo<D>::KK], float sl2e,
                                         GState<D>& st) {
    constexpr int kMode = TAIL ? kStepTail : kStepFull;
    GRegs<D> g;
    gqa_load<D, kMode>(kh, vh, kb, 0, e, w, c, g);
    __builtin_amdgcn_sched_barrier(0);   // all loads of the step in flight first
    gqa_compute<DT, D, kMode>(g, kb, 0, lim, w, qt, sl2e, st);
}

// Two full wave steps, keys [kb, kb + 32) and [kb + stride, +32): the loads of
// both in flight before either's arithmetic (twice the bytes in flight; at
// d = 128 this measured 8% slower than one step at a time).
template <int DT, int D>
__device__ __forceinline__ void gqa_step2(const char* __restrict__ kh, const char* __restrict__ vh,
                                          int kb, int stride, int w, int c,
                                          const u32x4_t (&qt)[GGeo<D>::KK], float sl2e,
                                          GState<D>& st) {
    GRegs<D> g0, g1;
    gqa_load<D, kStepFull>(kh, vh, kb, 0, 0, w, c, g0);
    gqa_load<D, kStepFull>(kh, vh, kb + stride, 0, 0, w, c, g1);
    __builtin_amdgcn_sched_barrier(0);
    gqa_compute<DT, D, kStepFull>(g0, kb, 0, 0, w, qt, sl2e, st);
    gqa_compute<DT, D, kStepFull>(g1, kb + stride, 0, 0, w, qt, sl2e, st);
}

// Stream keys [a, e) of one K/V head for the 16 query columns of qt. Keys
// below `full` (uniform) are seen by every column; this lane's column sees
// keys below lim (full <= lim <= e), which only the last steps test.
template <int DT, int D>
__device__ __forceinline__ void gqa_range(const uint16_t* kh, const uint16_t* vh, int a, int e,
                                          int full, int lim, int wave, int w, int c,
                                          const u32x4_t (&qt)[GGeo<D>::KK], float sl2e,
                                          GState<D>& st) {
    using G = GGeo<D>;
    const char* kc = reinterpret_cast<const char*>(kh);
    const char* vc = reinterpret_cast<const char*>(vh);
    int base = a;
    // d = 64: a step moves 8 KiB per wave; two steps' loads in flight at once
    // keep 16 KiB per wave in flight, like one step at d = 128
    if constexpr (D == 64)
        for (; base + 2 * G::CH <= full; base += 2 * G::CH)
            gqa_step2<DT, D>(kc, vc, base + G::KEYS * wave, G::CH, w, c, qt, sl2e, st);
    for (; base + G::CH <= full; base += G::CH)
        gqa_step<DT, D, false>(kc, vc, base + G::KEYS * wave, e, lim, w, c, qt, sl2e, st);
    for (; base < e; base += G::CH)
        gqa_step<DT, D, true>(kc, vc, base + G::KEYS * wave, e, lim, w, c, qt, sl2e, st);
}

// Q^T operands of a unit: lane (w, c) holds the query row of column c (row
// `row`, if live) at head-dim pieces w + 4kk; dead columns are zero.
template <int D>
__device__ __forceinline__ void load_qt(const uint16_t* q, int64_t row, bool live, int w,
                                        u32x4_t (&qt)[GGeo<D>::KK]) {
#pragma unroll
    for (int kk = 0; kk < GGeo<D>::KK; ++kk) {
        if (live)
            qt[kk] = *reinterpret_cast<const u32x4_t*>(
                reinterpret_cast<const char*>(q) +
                (uint64_t)(row * (int64_t)(D * 2) + (w + 4 * kk) * 16));
        else
            qt[kk] = u32x4_t{0u, 0u, 0u, 0u};
    }
}

template <int D>
struct alignas(16) GSmem {
    float o[kWaves][16][D + 4];   // padded rows: conflict-free float4 traffic
    float m[kWaves][16];
    float l[kWaves][16];
};

// Fold the waves' states with f. Thread t = 16*q + dc receives (M, L, O) of
// query column q for head dims [dc*DPT, dc*DPT + DPT).
template <int D>
__device__ __forceinline__ void gqa_fold(GSmem<D>& sm, GState<D>& st, int wave, int w, int c,
                                         float& M, float& L, float (&O)[GGeo<D>::DPT]) {
    using G = GGeo<D>;
    // the lanes of query c split its keys over w = 0..3: add their partial sums
    float l = st.l;
    l = sum_xor16_32(l);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int nb0 = 0; nb0 < G::NB; nb0 += 4) {
            float4 v = make_float4(st.o[nb0][r], st.o[nb0 + 1][r], st.o[nb0 + 2][r], st.o[nb0 + 3][r]);
            *reinterpret_cast<float4*>(&sm.o[wave][c][G::NB * (4 * w + r) + nb0]) = v;
        }
    }
    if (w == 0) {
        sm.m[wave][c] = st.m;
        sm.l[wave][c] = l;
    }
    __syncthreads();
    const int t = threadIdx.x;
    const int q = t >> 4;
    const int dc = t & 15;
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) mx = fmaxf(mx, sm.m[v][q]);
    const float mu = (mx == kNegInf) ? 0.f : mx;
    float ls = 0.f, o[G::DPT];
#pragma unroll
    for (int i = 0; i < G::DPT; ++i) o[i] = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const float wt = fexp2(sm.m[v][q] - mu);
        ls = fmaf(wt, sm.l[v][q], ls);
#pragma unroll
        for (int i0 = 0; i0 < G::DPT; i0 += 4) {
            const float4 x = *reinterpret_cast<const float4*>(&sm.o[v][q][dc * G::DPT + i0]);
            o[i0 + 0] = fmaf(wt, x.x, o[i0 + 0]);
            o[i0 + 1] = fmaf(wt, x.y, o[i0 + 1]);
            o[i0 + 2] = fmaf(wt, x.z, o[i0 + 2]);
            o[i0 + 3] = fmaf(wt, x.w, o[i0 + 3]);
        }
    }
    M = mx;
    L = ls;
#pragma unroll
    for (int i = 0; i < G::DPT; ++i) O[i] = o[i];
    __syncthreads();
}

struct Unit {
    int b, kvh, qb, geff;   // geff: live query columns of this block (<= 16)
    int64_t kvrow0;         // row of the K/V head's first key
    int n;
};

// A unit met through a lean segment: its request, length and token offset
// come with the segment.
__device__ __forceinline__ Unit decode_unit(const GqaArgs& a, const LeanSeg& s) {
    Unit x;
    x.b = s.b;
    x.kvh = s.unit / a.QB;
    x.qb = s.unit - x.kvh * a.QB;
    x.geff = min(16, a.cols - 16 * x.qb);
    x.n = s.n;
    x.kvrow0 = head_row0(a.kv_stride, a.Hk, x.b, x.kvh, s.tok_off, x.n);
    return x;
}

__device__ __forceinline__ Unit decode_unit(const GqaArgs& a, int u) {
    Unit x;
    const int upr = a.Hk * a.QB;
    x.b = u / upr;
    const int rem = u - x.b * upr;
    x.kvh = rem / a.QB;
    x.qb = rem - x.kvh * a.QB;
    x.geff = min(16, a.cols - 16 * x.qb);
    x.n = a.ctx[x.b];
    x.kvrow0 = head_row0(a.kv_stride, a.Hk, x.b, x.kvh, a.tok_off[x.b], x.n);
    return x;
}

// Row in q / out (and m_out / l_out) of live column c of a unit: column
// 16 qb + c is (query head hq of the group, token t), row (b Nq + t) H + kvh g + hq.
__device__ __forceinline__ int64_t col_row(const GqaArgs& a, const Unit& x, int c) {
    const int cg = 16 * x.qb + c;
    const int hq = cg / a.Nq;
    const int t = cg - hq * a.Nq;
    return ((int64_t)x.b * a.Nq + t) * a.H + (int64_t)x.kvh * a.g + hq;
}

// Keys column c sees: its token t sits at position n - Nq + t.
__device__ __forceinline__ int col_visible(const GqaArgs& a, const Unit& x, int c) {
    return x.n - a.Nq + 1 + (16 * x.qb + c) % a.Nq;
}

// Key bounds of a range [tok0, tok1) for lane column c: keys below `full` are
// seen by every column, keys below `lim` by column c.
__device__ __forceinline__ void col_bounds(const GqaArgs& a, const Unit& x, int c, int tok1,
                                           int& full, int& lim) {
    full = min(tok1, x.n - a.Nq + 1);
    lim = min(tok1, col_visible(a, x, c));
}

template <int D>
__device__ __forceinline__ void write_out_gqa(const GqaArgs& a, const Unit& x, int q, int dc,
                                              float M, float L, const float (&O)[GGeo<D>::DPT]) {
    if (q >= x.geff) return;
    const int64_t row = col_row(a, x, q);
    const float inv = 1.f / L;
    float* dst = a.out + row * D + dc * GGeo<D>::DPT;
#pragma unroll
    for (int i0 = 0; i0 < GGeo<D>::DPT; i0 += 4)
        *reinterpret_cast<float4*>(dst + i0) =
            make_float4(O[i0] * inv, O[i0 + 1] * inv, O[i0 + 2] * inv, O[i0 + 3] * inv);
    if (dc == 0) {
        if (a.m_out != nullptr) a.m_out[row] = M * kLn2;
        if (a.l_out != nullptr) a.l_out[row] = L;
    }
}

// Thread (q, dc)'s slice of peer p's record of column q: m, l and head dims
// [dc * DPT, +DPT) of Obar, loaded device-coherent.
template <int D>
__device__ __forceinline__ void load_rec_g(__amdgpu_buffer_rsrc_t xr, int p, int q, int dc,
                                           float& pm, float& pl, float (&po)[GGeo<D>::DPT]) {
    using G = GGeo<D>;
    const uint32_t rec = (uint32_t)(p * 16 + q) * (uint32_t)(part_stride(D) * 4);
    const float2 ml = load8_agent(xr, rec + (uint32_t)D * 4u);
    pm = ml.x;
    pl = ml.y;
#pragma unroll
    for (int i = 0; i < G::DPT; i += 4) {
        const float4 v = load16_agent(xr, rec + (uint32_t)(dc * G::DPT + i) * 4u);
        po[i] = v.x;
        po[i + 1] = v.y;
        po[i + 2] = v.z;
        po[i + 3] = v.w;
    }
}

// Host side of the lean exchange: fold the records of peers cta+1 .. last
// into thread (q, dc)'s state of column q, in ascending workgroup order, a
// batch of peers' loads in flight at a time (the streaming registers are free
// by now).
template <int D>
__device__ __forceinline__ void fold_peers(__amdgpu_buffer_rsrc_t xr, int cta, int last, int geff,
                                           int q, int dc, float& M, float& L,
                                           float (&O)[GGeo<D>::DPT]) {
    using G = GGeo<D>;
    constexpr int kBatch = 128 / D * 8;   // 16 peers at d = 64, 8 at d = 128
    for (int p0 = cta + 1; q < geff && p0 <= last; p0 += kBatch) {
        float pm[kBatch], pl[kBatch], po[kBatch][G::DPT];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            load_rec_g<D>(xr, min(p0 + j, last), q, dc, pm[j], pl[j], po[j]);
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (p0 + j <= last) merge_into<G::DPT>(M, L, O, pm[j], pl[j], po[j]);
    }
}

// The same for at most 4 live columns, whose records one wave alone would
// load: the live columns padded to Q (1, 2 or 4) leave R = 16 / Q thread
// groups per column. Group r folds peers cta+1+r, +R, +2R, ... of its column
// (group 0 onto the host's own state, the others from an empty one); then
// group 0 folds the other groups' states, in group order, through the first
// wave's slots of the fold area. All four waves load, so the merge runs at
// the CU's load rate (gqa-512k: 5.8 -> 3.3 us). Measured on 8 live columns
// (R = 2) the extra LDS round costs more than it saves. Used at d = 128: at
// d = 64 its registers would cost a wave per SIMD of occupancy.
template <int D>
__device__ __forceinline__ void fold_peers_spread(GSmem<D>& sm, __amdgpu_buffer_rsrc_t xr, int cta,
                                                  int last, int geff, int q, int dc, float& M,
                                                  float& L, float (&O)[GGeo<D>::DPT]) {
    using G = GGeo<D>;
    const int Q = geff <= 1 ? 1 : geff <= 2 ? 2 : 4;
    const int R = 16 / Q;
    const int r = q / Q;
    const int qc = q - r * Q;
    if (r > 0) {
        M = kNegInf;
        L = 0.f;
#pragma unroll
        for (int i = 0; i < G::DPT; ++i) O[i] = 0.f;
    }
    constexpr int kBatch = 8;   // peers per thread in flight (R >= 4 splits them)
    for (int p0 = cta + 1 + r; qc < geff && p0 <= last; p0 += kBatch * R) {
        float pm[kBatch], pl[kBatch], po[kBatch][G::DPT];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            load_rec_g<D>(xr, min(p0 + j * R, last), qc, dc, pm[j], pl[j], po[j]);
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (p0 + j * R <= last) merge_into<G::DPT>(M, L, O, pm[j], pl[j], po[j]);
    }
    // slot q (= r * Q + qc) of the first wave's fold area: group r's state of column qc
    if (r > 0 && qc < geff) {
#pragma unroll
        for (int i = 0; i < G::DPT; i += 4)
            *reinterpret_cast<float4*>(&sm.o[0][q][dc * G::DPT + i]) =
                make_float4(O[i], O[i + 1], O[i + 2], O[i + 3]);
        if (dc == 0) {
            sm.m[0][q] = M;
            sm.l[0][q] = L;
        }
    }
    __syncthreads();
    if (r == 0 && qc < geff) {
        for (int rr = 1; rr < R; ++rr) {
            const int s = rr * Q + qc;
            float po[G::DPT];
#pragma unroll
            for (int i = 0; i < G::DPT; i += 4) {
                const float4 v = *reinterpret_cast<const float4*>(&sm.o[0][s][dc * G::DPT + i]);
                po[i] = v.x;
                po[i + 1] = v.y;
                po[i + 2] = v.z;
                po[i + 3] = v.w;
            }
            merge_into<G::DPT>(M, L, O, sm.m[0][s], sm.l[0][s], po);
        }
    }
}

// ------------------------------------------------------------------ lean

// A lean segment whose streaming has begun: its unit, key range and bounds,
// the lane's query operands, where its step grid starts, and the kind of its
// first step. The first step's K/V loads sit in a GRegs issued with it.
template <int D>
struct GSeg {
    Unit x;
    int tok0, tok1, full, lim;
    int base0;      // first step's key: tok0, or up to one 4 KiB block of K before it
    int mode0;      // kStepFull, kStepTail or kStepEdge
    u32x4_t qt[GGeo<D>::KK];
};

// Set up segment `sg` and issue the loads of its first wave step into `g`.
// The step grid starts where the K rows cross a 4 KiB address boundary: each
// 16-key block of a wave's K loads (64 bytes of each of 16 rows per
// instruction) then covers whole 4 KiB blocks. Measured with a plain read of
// this load pattern at 4 GiB per K and V on MI355X, the rate depends on where
// a block starts: 7.22 TB/s aligned, down to 6.94 TB/s at 5-11 rows past a
// boundary. Packed caches put heads at arbitrary rows, so the grid is aligned
// here; the keys of the first step before tok0 are masked and their loads
// clamped into the segment. A segment shorter than kAlignMinSteps steps
// keeps its grid at tok0 where aligning would add a step: its time is the
// latency of its steps, not the rate of its reads.
template <int D>
__device__ __forceinline__ void gseg_start(const GqaArgs& a, const LeanSeg& sg, int wave, int w,
                                           int c, GSeg<D>& s, GRegs<D>& g) {
    using G = GGeo<D>;
    constexpr int kAlignRows = 4096 / G::RB;     // 16 at d = 128, 32 at d = 64
    s.x = decode_unit(a, sg);
    s.tok0 = sg.t0 * a.L;
    s.tok1 = (int)min((int64_t)sg.t1 * a.L, (int64_t)s.x.n);
    col_bounds(a, s.x, c, s.tok1, s.full, s.lim);
    const char* kc = reinterpret_cast<const char*>(a.k + s.x.kvrow0 * D);
    const char* vc = reinterpret_cast<const char*>(a.v + s.x.kvrow0 * D);
    const uint32_t phase =
        (uint32_t)(((uintptr_t)kc + (uint64_t)s.tok0 * G::RB) & 4095u) / G::RB;
    s.base0 = s.tok0 - (int)min(phase, (uint32_t)(kAlignRows - 1));
    if (s.tok1 - s.tok0 < kAlignMinSteps * G::CH &&
        (s.tok1 - s.base0 + G::CH - 1) / G::CH > (s.tok1 - s.tok0 + G::CH - 1) / G::CH)
        s.base0 = s.tok0;
    // uniform: full depends on the unit only
    s.mode0 = s.base0 < s.tok0 ? kStepEdge : (s.tok0 + G::CH > s.full ? kStepTail : kStepFull);
    load_qt<D>(a.q, c < s.x.geff ? col_row(a, s.x, c) : 0, c < s.x.geff, w, s.qt);
    const int kb = s.base0 + G::KEYS * wave;
    if (s.mode0 == kStepFull)
        gqa_load<D, kStepFull>(kc, vc, kb, s.tok0, s.tok1, w, c, g);
    else if (s.mode0 == kStepTail)
        gqa_load<D, kStepTail>(kc, vc, kb, s.tok0, s.tok1, w, c, g);
    else
        gqa_load<D, kStepEdge>(kc, vc, kb, s.tok0, s.tok1, w, c, g);
}

// Stream a started segment: its first step from the loaded `g`, then the rest.
template <int DT, int D>
__device__ __forceinline__ void gseg_stream(const GqaArgs& a, const GSeg<D>& s, const GRegs<D>& g,
                                            int wave, int w, int c, GState<D>& st) {
    using G = GGeo<D>;
    const int kb = s.base0 + G::KEYS * wave;
    if (s.mode0 == kStepFull)
        gqa_compute<DT, D, kStepFull>(g, kb, s.tok0, s.lim, w, s.qt, a.sl2e, st);
    else if (s.mode0 == kStepTail)
        gqa_compute<DT, D, kStepTail>(g, kb, s.tok0, s.lim, w, s.qt, a.sl2e, st);
    else
        gqa_compute<DT, D, kStepEdge>(g, kb, s.tok0, s.lim, w, s.qt, a.sl2e, st);
    gqa_range<DT, D>(a.k + s.x.kvrow0 * D, a.v + s.x.kvrow0 * D, s.base0 + G::CH, s.tok1, s.full,
                     s.lim, wave, w, c, s.qt, a.sl2e, st);
}

// Segments of a workgroup are streamed back to back: when one ends, the next
// one's query operands and first K/V step are loaded before the cross-wave
// fold and the epilogue of the one that ended, so that their latency overlaps
// that work instead of stalling every wave at the start of the next segment.
// A host that merges its peers' records loads the next segment after the
// merge, whose batched record loads need those registers.
template <int DT, int D, int SRC>
__global__ __launch_bounds__(kThreads, 2) void lean_gqa_kernel(const GqaArgs a) {
    using G = GGeo<D>;
    __shared__ GSmem<D> sm;
    const int cta = blockIdx.x;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int w = (t >> 4) & 3;
    const int c = t & 15;
    const int q = t >> 4;
    const int dc = t & 15;
    const __amdgpu_buffer_rsrc_t xr = exchange_rsrc(a.part, a.part_bytes);
    const uint64_t t_in = stamp_start(a.ts, cta);
    const uint32_t ep = launch_epoch(a.ctl);
    __shared__ SchedLds sl;
    SegCursor<SRC> cur(a.sched, kernarg_sched<GqaArgs>(), sl, cta);
    if (cur.bad()) {   // lengths from device memory out of range: nothing is computed
        if (cta == 0 && t == 0) atomicOr(&a.ctl[kCtlErr], kErrLengths);
        if (t == 0) launch_exit(a.ctl, ep);
        stamp_end(a.ts, cta);
        return;
    }
    LeanSeg sg;
    bool have = cur.next(sg);
    GSeg<D> cs;
    GRegs<D> pre;
    if (have) gseg_start<D>(a, sg, wave, w, c, cs, pre);
    while (have) {
        GState<D> st;
        gstate_init<D>(st);
        gseg_stream<DT, D>(a, cs, pre, wave, w, c, st);
        if (a.tile_owner != nullptr && t == 0)
            for (int i = sg.t0; i < sg.t1; ++i) a.tile_owner[sg.iter0 + i - sg.t0] = cta;

        LeanSeg nsg;
        const bool nhave = cur.next(nsg);
        const bool merging = sg.host && !sg.fin;
        GSeg<D> ns;
        if (nhave && !merging) gseg_start<D>(a, nsg, wave, w, c, ns, pre);

        float M, L, O[G::DPT];
        gqa_fold<D>(sm, st, wave, w, c, M, L, O);

        if (!sg.host) {
            // a peer: publish one record per query column, then raise the
            // flag to this launch's epoch
            if (q < cs.x.geff) {
                const uint32_t rec = (uint32_t)(cta * 16 + q) * (uint32_t)(part_stride(D) * 4);
#pragma unroll
                for (int i = 0; i < G::DPT; i += 4)
                    store16_agent(xr, rec + (uint32_t)(dc * G::DPT + i) * 4u,
                                  make_float4(O[i], O[i + 1], O[i + 2], O[i + 3]));
                if (dc == 0) store8_agent(xr, rec + (uint32_t)D * 4u, M, L);
            }
            drain_stores();
            __syncthreads();
            if (t == 0) __hip_atomic_store(&a.flags[cta], ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (merging) {
                // the host: wait for every peer at once, then fold their records
                const int last = sg.last;
                const int np = last - cta;
                const uint64_t w0 = stamp_now(a.ts);
                for (int i = t; i < np; i += kThreads)
                    wait_flag(&a.flags[cta + 1 + i], ep, a.wait_ticks, a.ctl);
                __syncthreads();
                stamp_wait(a.ts, cta, t_in, w0);
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                // The host's CU reads every peer's records, so the merge runs
                // at one CU's load rate; with at most 4 live columns the idle
                // column groups share the loads.
                if (D == 128 && cs.x.geff <= 4)
                    fold_peers_spread<D>(sm, xr, cta, last, cs.x.geff, q, dc, M, L, O);
                else
                    fold_peers<D>(xr, cta, last, cs.x.geff, q, dc, M, L, O);
            }
            write_out_gqa<D>(a, cs.x, q, dc, M, L, O);
            if (nhave && merging) gseg_start<D>(a, nsg, wave, w, c, ns, pre);
        }
        sg = nsg;
        cs = ns;
        have = nhave;
    }
    if (t == 0) launch_exit(a.ctl, ep);
    stamp_end(a.ts, cta);
}

// ------------------------------------------------------------------ dynamic pull

// Slot of a unit's piece in chunk ch: (ch, 0) if the piece starts the chunk,
// else (ch, 1). A slot holds 16 records, one per query column.
__device__ __forceinline__ int piece_slot_g(int ch, int Su, int C) {
    return ch * 2 + (max(Su, ch * C) == ch * C ? 0 : 1);
}

__device__ __forceinline__ uint32_t rec_off(int slot, int q, int D) {
    return (uint32_t)(slot * 16 + q) * (uint32_t)(part_stride(D) * 4);
}

// Thread (q, dc) stores its slice of column q's record of `slot`.
template <int D>
__device__ __forceinline__ void publish_rec_g(__amdgpu_buffer_rsrc_t xr, int slot, int q, int dc,
                                              int geff, float M, float L,
                                              const float (&O)[GGeo<D>::DPT]) {
    using G = GGeo<D>;
    if (q >= geff) return;
    const uint32_t rec = rec_off(slot, q, D);
#pragma unroll
    for (int i = 0; i < G::DPT; i += 4)
        store16_agent(xr, rec + (uint32_t)(dc * G::DPT + i) * 4u,
                      make_float4(O[i], O[i + 1], O[i + 2], O[i + 3]));
    if (dc == 0) store8_agent(xr, rec + (uint32_t)D * 4u, M, L);
}

// Workgroup-wide: once every wave's record stores have completed, add one to
// the counter; true in every thread when that add was the last (`last` + 1).
__device__ __forceinline__ bool count_in_wg(uint32_t* ctr, int last, int& s_word) {
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        s_word = (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool mine = s_word == last;
    __syncthreads();   // s_word is read by all before it can be written again
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return mine;
}

// Fold, in order, column qq's records of chunks ch0, ch0 + step, ... (n of
// them) at slot level `lvl` into (M, L, O), replacing what they held. Callers
// skip columns past the group (their records were never written).
template <int D>
__device__ __forceinline__ void fold_slots_g(__amdgpu_buffer_rsrc_t xr, int lvl, int ch0, int n,
                                             int step, int Su, int C, int qq, int dc, float& M,
                                             float& L, float (&O)[GGeo<D>::DPT]) {
    using G = GGeo<D>;
    constexpr int kBatch = 128 / D * 8;   // 16 records in flight at d = 64, 8 at d = 128
    M = kNegInf;
    L = 0.f;
#pragma unroll
    for (int i = 0; i < G::DPT; ++i) O[i] = 0.f;
    for (int i0 = 0; i0 < n; i0 += kBatch) {
        float pm[kBatch], pl[kBatch], po[kBatch][G::DPT];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int ch = ch0 + min(i0 + j, n - 1) * step;
            const uint32_t rec = rec_off(lvl + piece_slot_g(ch, Su, C), qq, D);
            const float2 ml = load8_agent(xr, rec + (uint32_t)D * 4u);
            pm[j] = ml.x;
            pl[j] = ml.y;
#pragma unroll
            for (int i = 0; i < G::DPT; i += 4) {
                const float4 v = load16_agent(xr, rec + (uint32_t)(dc * G::DPT + i) * 4u);
                po[j][i] = v.x;
                po[j][i + 1] = v.y;
                po[j][i + 2] = v.z;
                po[j][i + 3] = v.w;
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (i0 + j < n) merge_into<G::DPT>(M, L, O, pm[j], pl[j], po[j]);
    }
}

// Chunks of the unit tile sequence, taken from an atomic counter (dynamic) or
// one per workgroup; a unit spread over chunks leaves 16 records (one per
// query column) per chunk at slot (chunk, side), and the workgroup whose
// piece arrives last merges them in chunk order. Nothing waits.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void pull_gqa_kernel(const GqaArgs a) {
    using G = GGeo<D>;
    __shared__ GSmem<D> sm;
    __shared__ int s_chunk, s_arrived;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int w = (t >> 4) & 3;
    const int c = t & 15;
    const int q = t >> 4;
    const int dc = t & 15;
    const __amdgpu_buffer_rsrc_t xr = exchange_rsrc(a.part, a.part_bytes);
    stamp_start(a.ts, blockIdx.x);
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
            const Unit x = decode_unit(a, u);
            const int tok0 = (it - Su) * a.L;
            const int tok1 = (int)min((int64_t)(t1 - Su) * a.L, (int64_t)x.n);
            u32x4_t qt[G::KK];
            load_qt<D>(a.q, c < x.geff ? col_row(a, x, c) : 0, c < x.geff, w, qt);
            int full, lim;
            col_bounds(a, x, c, tok1, full, lim);
            GState<D> st;
            gstate_init<D>(st);
            gqa_range<DT, D>(a.k + x.kvrow0 * D, a.v + x.kvrow0 * D, tok0, tok1, full, lim, wave,
                             w, c, qt, a.sl2e, st);
            if (a.tile_owner != nullptr)
                for (int i = it + t; i < t1; i += kThreads) a.tile_owner[i] = blockIdx.x;
            float M, L, O[G::DPT];
            gqa_fold<D>(sm, st, wave, w, c, M, L, O);
            const int side = it == c0 ? 0 : 1;
            it = t1;
            const int kf = Su / a.C, kl = (Se - 1) / a.C;   // chunks holding unit u
            if (kf != kl) {
                // two-level merge tree over the unit's chunks (groups of
                // kMergeFanIn), as in the single-head pull kernel
                const int g0 = kf + (k - kf) / kMergeFanIn * kMergeFanIn;
                const int g1 = min(g0 + kMergeFanIn - 1, kl);
                const int ngroups = (kl - kf) / kMergeFanIn + 1;
                const int gslot = piece_slot_g(g0, Su, a.C);
                if (g1 > g0) {
                    publish_rec_g<D>(xr, k * 2 + side, q, dc, x.geff, M, L, O);
                    if (!count_in_wg(&a.gcount[gslot], g1 - g0, s_arrived)) continue;
                    if (q < x.geff)
                        fold_slots_g<D>(xr, 0, g0, g1 - g0 + 1, 1, Su, a.C, q, dc, M, L, O);
                    if (t == 0)
                        __hip_atomic_store(&a.gcount[gslot], 0u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                if (ngroups > 1) {
                    const int l1 = 2 * a.nchunks;   // second-level slots follow the first
                    publish_rec_g<D>(xr, l1 + gslot, q, dc, x.geff, M, L, O);
                    if (!count_in_wg(&a.arrive[u], ngroups - 1, s_arrived)) continue;
                    if (q < x.geff)
                        fold_slots_g<D>(xr, l1, kf, ngroups, kMergeFanIn, Su, a.C, q, dc, M, L,
                                        O);
                    if (t == 0)
                        __hip_atomic_store(&a.arrive[u], 0u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            write_out_gqa<D>(a, x, q, dc, M, L, O);
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
    if (a.dynamic && t == 0) {
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
__global__ __launch_bounds__(kThreads) void split_gqa_kernel(const GqaArgs a) {
    using G = GGeo<D>;
    __shared__ GSmem<D> sm;
    stamp_start(a.ts, blockIdx.x);
    const int u = blockIdx.x / a.splits;
    const int k = blockIdx.x - u * a.splits;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int w = (t >> 4) & 3;
    const int c = t & 15;
    const Unit x = decode_unit(a, u);
    const int64_t T = ((int64_t)x.n + a.L - 1) / a.L;
    const int64_t t0 = (int64_t)k * T / a.splits, t1 = (int64_t)(k + 1) * T / a.splits;
    const int tok0 = (int)(t0 * a.L);
    const int tok1 = (int)min(t1 * a.L, (int64_t)x.n);
    u32x4_t qt[G::KK];
    load_qt<D>(a.q, c < x.geff ? col_row(a, x, c) : 0, c < x.geff, w, qt);
    int full, lim;
    col_bounds(a, x, c, tok1, full, lim);
    GState<D> st;
    gstate_init<D>(st);
    if (tok0 < tok1)
        gqa_range<DT, D>(a.k + x.kvrow0 * D, a.v + x.kvrow0 * D, tok0, tok1, full, lim, wave, w,
                         c, qt, a.sl2e, st);
    float M, L, O[G::DPT];
    gqa_fold<D>(sm, st, wave, w, c, M, L, O);
    const int q = t >> 4, dc = t & 15;
    if (q < x.geff) {
        float* p = a.part + ((int64_t)blockIdx.x * 16 + q) * part_stride(D);
#pragma unroll
        for (int i = 0; i < G::DPT; ++i) p[dc * G::DPT + i] = O[i];
        if (dc == 0) {
            p[D] = M;
            p[D + 1] = L;
        }
    }
    stamp_end(a.ts, blockIdx.x);
}

// One wave per (unit, query column): folds the unit's `splits` records in order.
template <int D>
__global__ __launch_bounds__(64) void combine_gqa_kernel(const GqaArgs a) {
    constexpr int P = D / 64;
    const int u = blockIdx.x >> 4;
    const int q = blockIdx.x & 15;
    const int lane = threadIdx.x;
    const Unit x = decode_unit(a, u);
    if (q >= x.geff) return;
    float M = kNegInf, L = 0.f, O[P];
#pragma unroll
    for (int j = 0; j < P; ++j) O[j] = 0.f;
    for (int k = 0; k < a.splits; ++k) {
        const float* p = a.part + (((int64_t)u * a.splits + k) * 16 + q) * part_stride(D);
        float po[P];
#pragma unroll
        for (int j = 0; j < P; ++j) po[j] = p[lane + 64 * j];
        merge_into<P>(M, L, O, p[D], p[D + 1], po);
    }
    const int64_t row = col_row(a, x, q);
    const float inv = 1.f / L;
#pragma unroll
    for (int j = 0; j < P; ++j) a.out[row * D + lane + 64 * j] = O[j] * inv;
    if (lane == 0) {
        if (a.m_out != nullptr) a.m_out[row] = M * kLn2;
        if (a.l_out != nullptr) a.l_out[row] = L;
    }
}

// ------------------------------------------------------------------ per head

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void per_head_gqa_kernel(const GqaArgs a) {
    using G = GGeo<D>;
    __shared__ GSmem<D> sm;
    stamp_start(a.ts, blockIdx.x);
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int w = (t >> 4) & 3;
    const int c = t & 15;
    const Unit x = decode_unit(a, blockIdx.x);
    u32x4_t qt[G::KK];
    load_qt<D>(a.q, c < x.geff ? col_row(a, x, c) : 0, c < x.geff, w, qt);
    int full, lim;
    col_bounds(a, x, c, x.n, full, lim);
    GState<D> st;
    gstate_init<D>(st);
    gqa_range<DT, D>(a.k + x.kvrow0 * D, a.v + x.kvrow0 * D, 0, x.n, full, lim, wave, w, c, qt,
                     a.sl2e, st);
    float M, L, O[G::DPT];
    gqa_fold<D>(sm, st, wave, w, c, M, L, O);
    write_out_gqa<D>(a, x, t >> 4, t & 15, M, L, O);
    stamp_end(a.ts, blockIdx.x);
}

template <typename F>
const void* pick_g(int dtype, int d, F f16_64, F f16_128, F bf16_64, F bf16_128) {
    if (dtype == 0) return d == 64 ? (const void*)f16_64 : (const void*)f16_128;
    return d == 64 ? (const void*)bf16_64 : (const void*)bf16_128;
}

}  // namespace

const void* lean_gqa_kernel_ptr(int dtype, int d, int src) {
    if (src == kSrcArgs)
        return pick_g(dtype, d, &lean_gqa_kernel<0, 64, kSrcArgs>,
                      &lean_gqa_kernel<0, 128, kSrcArgs>, &lean_gqa_kernel<1, 64, kSrcArgs>,
                      &lean_gqa_kernel<1, 128, kSrcArgs>);
    if (src == kSrcDevice)
        return pick_g(dtype, d, &lean_gqa_kernel<0, 64, kSrcDevice>,
                      &lean_gqa_kernel<0, 128, kSrcDevice>, &lean_gqa_kernel<1, 64, kSrcDevice>,
                      &lean_gqa_kernel<1, 128, kSrcDevice>);
    return pick_g(dtype, d, &lean_gqa_kernel<0, 64, kSrcTables>,
                  &lean_gqa_kernel<0, 128, kSrcTables>, &lean_gqa_kernel<1, 64, kSrcTables>,
                  &lean_gqa_kernel<1, 128, kSrcTables>);
}

hipError_t launch_lean_gqa(int dtype, int d, const GqaArgs& a, int grid, hipStream_t s,
                           bool cooperative) {
    const void* fn = lean_gqa_kernel_ptr(dtype, d, a.sched.src);
    void* args[] = {const_cast<GqaArgs*>(&a)};
    if (cooperative)
        return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_pull_gqa(int dtype, int d, const GqaArgs& a, int grid, hipStream_t s) {
    const void* fn = pick_g(dtype, d, &pull_gqa_kernel<0, 64>, &pull_gqa_kernel<0, 128>,
                            &pull_gqa_kernel<1, 64>, &pull_gqa_kernel<1, 128>);
    void* args[] = {const_cast<GqaArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_split_gqa(int dtype, int d, const GqaArgs& a, int blocks, hipStream_t s) {
    const void* fn = pick_g(dtype, d, &split_gqa_kernel<0, 64>, &split_gqa_kernel<0, 128>,
                            &split_gqa_kernel<1, 64>, &split_gqa_kernel<1, 128>);
    void* args[] = {const_cast<GqaArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(blocks), dim3(kThreads), args, 0, s);
}

hipError_t launch_combine_gqa(int d, const GqaArgs& a, int units, hipStream_t s) {
    const void* fn =
        d == 64 ? (const void*)&combine_gqa_kernel<64> : (const void*)&combine_gqa_kernel<128>;
    void* args[] = {const_cast<GqaArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(units * 16), dim3(64), args, 0, s);
}

hipError_t launch_per_head_gqa(int dtype, int d, const GqaArgs& a, int units, hipStream_t s) {
    const void* fn = pick_g(dtype, d, &per_head_gqa_kernel<0, 64>, &per_head_gqa_kernel<0, 128>,
                            &per_head_gqa_kernel<1, 64>, &per_head_gqa_kernel<1, 128>);
    void* args[] = {const_cast<GqaArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(units), dim3(kThreads), args, 0, s);
}

}  // namespace la
