// Whole-head, time-segmented inter-chunk state carry (gfx950).
//
// The carry of the chunkwise WY/UT prefill (ExecuTorch PR #21021 "Reorder channelwise gated
// delta rule chunked hot loops for autovectorization", second commit summary: WY
// pseudo-keys/values and inter-chunk state carry) advances the state S (dk x dv) chunk by
// chunk with the operands chunk_prep wrote to the workspace:
//   U  = Tb V - W S,   O = Qt S + P U,   S' = diag(exp(gam_last)) S + Kb^T U.
// For a fixed chunk this map is affine in S, so a run of chunks (a segment) is too:
//   S_end = M S_start + S_loc,
// where M is what the recurrence does to S_start with V = 0 (start from the identity) and
// S_loc is what it produces from S_start = 0.  The sequence is cut into NSEG segments:
//   1. carry_wide_kernel<SUM = true>: every segment but the last, in parallel, runs the
//      recurrence without outputs on the augmented state [S_loc | M] (from [0 | I]);
//   2. carry_combine_kernel: per head, S_start of segment s + 1 = M_s S_start(s) + S_loc_s
//      (fp16 hi/lo split operands, three matrix-core products per term: ~22-bit operands);
//   3. carry_wide_kernel<SUM = false>: every segment, in parallel, runs the full recurrence
//      from its start state and writes the outputs (the last one also the final state).
// With a single segment only step 3 runs, from h0.
//
// One workgroup owns a whole head (all dv columns) for its segment, so every byte of a
// chunk record is fetched from memory once per head: the record is staged into LDS by
// LDS-DMA loads (two buffers; the next chunk's copy is issued at the start of each step,
// and since each wave picks its copy slots at run time the compiler makes the step's first
// LDS read wait for that copy, so copy and compute take turns -- with many heads the pass
// runs at the HBM rate regardless), and each wave owns 16*CTW columns of the state for
// all dk rows.  A wave therefore computes every row
// of U and O for its columns and needs no operand from another wave: the only workgroup
// synchronisation is one barrier per chunk for the staged record.  Accumulator tiles of
// S and U feed the B operands of the next products directly (reduction slots follow
// perm_slot); v is transposed through a wave-private LDS tile.
//
// Range.  Each wave keeps its state columns in a scaled domain X' = X 2^-E (E per wave):
// per chunk it checks the largest magnitude of X' against fp16's comfortable range and,
// when it leaves it, moves E (an exact power-of-two rescale of X').  v enters the products
// as V 2^-EV with its own per-chunk exponent EV, so a state far smaller than v (or the
// reverse) keeps its precision; Tb V and W X meet in fp32 at EU = max(E, EV), U is
// published at 2^-EU and the state moves to that domain with the update (2^(E - EU) is
// folded into the decay factors).  O is 2^E Qt X' + 2^EU P U times the query rows' record
// multipliers (see chunk_prep); the final state (or segment summary) is X' 2^E.  So every
// fp16 operand stays inside fp16's range for state and v magnitudes within fp32's normal
// range; U itself keeps fp16's precision while beta >= 2^-12 (or beta = 0 exactly).
#include "gdr_device.h"
#include "gdr_launch.h"
#include "gdr_stage.h"

namespace gdr {
namespace {

typedef _Float16 half4w __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4w h4(f32x4 x) {
    return half4w{static_cast<_Float16>(x[0]), static_cast<_Float16>(x[1]), static_cast<_Float16>(x[2]),
                  static_cast<_Float16>(x[3])};
}
__device__ __forceinline__ half8 cat(half4w a, half4w b) {
    return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The copy list padded to a whole number of entries per wave: the extra entries copy the
// decay block once more into a spare slot, so every wave issues the same copies with no
// per-wave branch.
template <int C, int D, bool SUM, int NWAVE>
constexpr CopyList make_padded_list() {
    CopyList l = make_copy_list<C, D, SUM>();
    const int id = l.id[l.n - 1];
    const int spare = Stage<C, D, SUM>::nslot;
    while (l.n % NWAVE) {
        l.id[l.n] = (short)id;
        l.slot[l.n] = (short)spare;
        ++l.n;
    }
    return l;
}

// Entry `J * NWAVE + w` of the padded copy list, with w wave-uniform: a chain of scalar
// selects over compile-time entries (no indexed table in memory, no branch).
template <int NWAVE, int J, int C, int D, bool SUM>
__device__ __forceinline__ void copy_entry(int w, int& id, int& slot) {
    constexpr CopyList L = make_padded_list<C, D, SUM, NWAVE>();
    id = L.id[J * NWAVE];
    slot = L.slot[J * NWAVE];
#pragma unroll
    for (int ww = 1; ww < NWAVE; ++ww) {
        if (w == ww) {
            id = L.id[J * NWAVE + ww];
            slot = L.slot[J * NWAVE + ww];
        }
    }
}

// Segment s of NSEG covers chunks [s * NC / NSEG, (s + 1) * NC / NSEG).
__device__ __forceinline__ int seg_begin(int s, int NC, int NSEG) {
    return (int)(((long long)s * NC) / NSEG);
}

// SUM = false: full carry of one segment (outputs; final state from the last segment).
// SUM = true : waves 0..3 carry S_loc (from zero, with v), waves 4..7 carry M (from the
//              identity, without v); both are written to `xsum` at the segment's end.
// The staged records fill most of the LDS, so one workgroup runs per CU (full pass: one wave
// per SIMD; summary pass: two); the attribute states that occupancy to the compiler.
template <typename TIn, int D, int C, bool SUM, bool OBF = false>
__global__ __launch_bounds__(SUM ? 512 : 256) __attribute__((amdgpu_waves_per_eu(SUM ? 2 : 1, SUM ? 2 : 1)))
void carry_wide_kernel(
    const TIn* __restrict__ v, const float* h0, void* __restrict__ o, float* ht,
    const unsigned char* __restrict__ ws, float* xsum, const float* sstart, int B, int T,
    int HV, int NCD, int NSEG, const int32_t* __restrict__ plan) {
    constexpr int obf = OBF;  // o stored as bf16 (a compile-time choice: no branch per store)
    using ST = Stage<C, D, SUM>;
    constexpr ChunkRecord R = ST::R;
    constexpr int NB = ST::NB, NQS = ST::NQS, KC = ST::KC, DKT = ST::DKT;
    constexpr int NWAVE = SUM ? 8 : 4;
    constexpr int CTW = D / 64;                 // 16-column tiles per wave
    constexpr CopyList CL = make_copy_list<C, D, SUM>();
    constexpr int NCOPY = (CL.n + NWAVE - 1) / NWAVE;  // record fragments copied per wave
    constexpr int ELT = sizeof(TIn);
    constexpr int VP = C + 4;                   // padded token stride of the v tile
    constexpr int VLD = 16 * CTW * ELT / 16;    // 16-byte v loads per lane (one token row)

    __shared__ half8 sRec[2][(ST::nslot + 1) * 64];  // + the spare slot of the padded copy list
    __shared__ __attribute__((aligned(16))) _Float16 sV[4][16 * CTW * VP];

    const int NH = B * HV;
    const int bh = blockIdx.x % NH;
    const int seg = blockIdx.x / NH;
    const int h = bh % HV;
    const int b = bh / HV;
    // this batch element's (or packed sequence's) rows, chunks and first chunk slot; a packed
    // batch runs as one segment (NSEG = 1)
    const SeqSpan sp = seq_span(plan, b, B, T, NCD);
    const int NC = sp.nc;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int part = SUM ? (w >> 2) : 0;        // 0: state (with v), 1: transition M
    const int wq = w & 3;
    const int col0 = 16 * CTW * wq;             // first column of this wave
    const bool has_v = part == 0;

    const int c0 = seg_begin(seg, NC, NSEG);
    const int c1 = seg_begin(seg + 1, NC, NSEG);

    // state tiles in accumulator layout: X[rt][ct][i] = X[16 rt + 4 gq + i][col0 + 16 ct + li]
    f32x4 X[DKT][CTW];
    {
        const float* src = nullptr;
        if (!SUM) src = NSEG > 1 ? sstart + (size_t)(bh * NSEG + seg) * D * D : (h0 ? h0 + (size_t)bh * D * D : nullptr);
#pragma unroll
        for (int rt = 0; rt < DKT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                const int col = col0 + 16 * ct + li;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rt + 4 * gq + i;
                    if (SUM) x[i] = (part == 1 && row == col) ? 1.f : 0.f;
                    else if (src) x[i] = src[(size_t)row * D + col];
                }
                X[rt][ct] = x;
            }
    }

    // this wave's scaled domain: X' = X 2^-E (E wave-uniform; kNoExp while X and v are zero)
    auto max_abs_x = [&]() {
        float m = 0.f;
#pragma unroll
        for (int rt = 0; rt < DKT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(X[rt][ct][i]));
        return wave_max(m);
    };
    auto rescale_x = [&](int d) {  // X' *= 2^d
#pragma unroll
        for (int rt = 0; rt < DKT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[rt][ct][i] = ldexp2(X[rt][ct][i], d);
    };
    int E = kNoExp;
    {
        const float m = max_abs_x();
        if (m > 0.f) {
            E = __builtin_amdgcn_readfirstlane(exponent_of(m) - kTop);
            rescale_x(-E);
        }
    }

    const unsigned char* rec0 = ws + ((size_t)sp.c0 * HV + (size_t)h * NC) * R.bytes;
    const rsrc_t rs_rec = make_rsrc(rec0, (uint32_t)NC * R.bytes);
    const int rowv = HV * D * ELT;
    const int rowo = HV * D * o_elt(obf);
    const rsrc_t rs_v = make_rsrc(v + (size_t)sp.row0 * HV * D, (uint32_t)sp.T * rowv);
    const rsrc_t rs_o =
        make_rsrc(static_cast<unsigned char*>(o) + (size_t)sp.row0 * rowo, (uint32_t)sp.T * rowo);

    // Record staging: each wave copies its share of the copy list straight from memory into
    // the LDS buffer with LDS-DMA loads (16 bytes per lane, no registers); the copy of chunk
    // n + 1 is issued at the start of chunk n's step and waited for (vmcnt) before the next
    // barrier (the compiler also waits for it before the step's first LDS read).
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue_rec = [&](int n, int buf) {
#define GDR_LD(J)                                                                                  \
    if constexpr (J < NCOPY) {                                                                    \
        int id, slot;                                                                             \
        copy_entry<NWAVE, J, C, D, SUM>(w, id, slot);                                             \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_rec, (lds_void*)&sRec[buf][slot * 64], 16,      \
                                                 lane * 16, n * R.bytes + id * 1024, 0, 0);        \
    }
        GDR_LD(0) GDR_LD(1) GDR_LD(2) GDR_LD(3) GDR_LD(4) GDR_LD(5) GDR_LD(6) GDR_LD(7)
        GDR_LD(8) GDR_LD(9) GDR_LD(10) GDR_LD(11) GDR_LD(12) GDR_LD(13) GDR_LD(14) GDR_LD(15)
        GDR_LD(16) GDR_LD(17) GDR_LD(18) GDR_LD(19) GDR_LD(20) GDR_LD(21) GDR_LD(22) GDR_LD(23)
#undef GDR_LD
    };
    static_assert(NCOPY <= 24, "copy list share exceeds the unrolled staging slots");
    // wait for this wave's outstanding vector-memory operations (LDS-DMA copies, v loads,
    // output stores), all issued at the start of the chunk step
    auto wait_vm = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
        asm volatile("" ::: "memory");
    };

    // v rows of a chunk: lane t < C loads token t's 16*CTW columns of this wave (raw bits);
    // rows past T lie beyond the buffer range and read as zero.
    typedef u32x4 VRegs[VLD];
    auto issue_v = [&](VRegs& VR, int n) {
        if (!has_v) return;
        // lanes past the chunk length read from beyond the range (zeros, no memory access)
        const int off = lane < C ? ((n * C + lane) * HV + h) * D * ELT + col0 * ELT : (int)0xFFFFFF00u;
#pragma unroll
        for (int j = 0; j < VLD; ++j) {
            VR[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_v, off + 16 * j, 0, 0));
            asm volatile("" ::: "memory");
        }
    };
    auto publish_v = [&](const VRegs& VR, int E) {  // -> sV[wq][col][token], fp16 * 2^-E
        if (!has_v || lane >= C) return;
        _Float16* dst = sV[wq];
#pragma unroll
        for (int j = 0; j < VLD; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ELT == 2) {
                    const uint32_t u = VR[j][e];
                    dst[(8 * j + 2 * e) * VP + lane] = static_cast<_Float16>(ldexp2(__uint_as_float(u << 16), -E));
                    dst[(8 * j + 2 * e + 1) * VP + lane] =
                        static_cast<_Float16>(ldexp2(__uint_as_float(u & 0xFFFF0000u), -E));
                } else {
                    dst[(4 * j + e) * VP + lane] = static_cast<_Float16>(ldexp2(__uint_as_float(VR[j][e]), -E));
                }
            }
    };
    // outputs of chunk n, stored at the start of the next chunk step: lane (i, g) holds token
    // 16r + i, columns col0 + 16ct + 4g .. +3; rows past T are beyond the range and dropped
    f32x4 Oq[NB][CTW];
    // (on = false: the offset is beyond the range and the stores are dropped)
    auto store_o = [&](int n, bool on) {
        if constexpr (!SUM) {
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                const int obase = on ? ((n * C + 16 * r + li) * HV + h) * D * 4 + (col0 + 4 * gq) * 4
                                     : (int)0xFFFFFF00u;
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) store_o4_stream(Oq[r][ct], rs_o, obase, ct * 64, obf);
            }
        }
    };

    // One chunk step: v of chunk n to LDS, chunk n + 1's v and record requested, chunk n - 1's
    // outputs stored, chunk n computed from LDS buffer `buf`.
    VRegs VR;
    // The last step requests its own chunk again (clamped index) rather than branching.
    auto step = [&](int n, int buf) {
        const int nn = min(n + 1, c1 - 1);
        // keep X' at most 2^kTop and not far below it; this chunk's v at 2^-EV, its maximum
        // in [2^(kTop-1), 2^kTop)
        int EV = kNoExp;
        {
            VMax<TIn> vm;
            if (has_v) {
#pragma unroll
                for (int j = 0; j < VLD; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) vm.add(VR[j][e]);
            }
            const float mv = wave_max(vm.get());
            EV = __builtin_amdgcn_readfirstlane(mv > 0.f ? exponent_of(mv) - kTop : kNoExp);
            const float mx = E != kNoExp ? max_abs_x() : 0.f;
            if (mx > 0.f) {
                const int en = __builtin_amdgcn_readfirstlane(exponent_of(mx) + E - kTop);
                if (en > E || en < E - kSlack) {
                    rescale_x(E - en);
                    E = en;
                }
            } else {
                E = kNoExp;  // X' is zero
            }
        }
        const int EU = max(E, EV);
        publish_v(VR, EV);
        issue_v(VR, nn);
        lds_barrier();  // buffer `buf` complete; everyone is done with buffer buf ^ 1
        issue_rec(nn, buf ^ 1);
        store_o(n - 1, n > c0);

        const half8* L = sRec[buf];
        auto A = [&](int slot) { return L[slot * 64 + lane]; };

        // B fragments of the state (rows 32p .. 32p+31 = tiles 2p, 2p+1)
        half8 XB[KC][CTW];
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) XB[p][ct] = cat(h4(X[2 * p][ct]), h4(X[2 * p + 1][ct]));

        // U = Tb V - W X, the two products at their own scales, combined in fp32 at 2^-EU
        f32x4 U[NB][CTW], UX[NB][CTW];
#pragma unroll
        for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) U[r][ct] = UX[r][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (has_v) {
            half8 Vb[NQS][CTW];
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) {
                    const _Float16* colp = &sV[wq][(16 * ct + li) * VP + 32 * qs + 4 * gq];
                    const half4w lo = *reinterpret_cast<const half4w*>(colp);
                    half4w hi = {static_cast<_Float16>(0.f), static_cast<_Float16>(0.f),
                                 static_cast<_Float16>(0.f), static_cast<_Float16>(0.f)};
                    if (32 * qs + 16 < C) hi = *reinterpret_cast<const half4w*>(colp + 16);
                    Vb[qs][ct] = cat(lo, hi);
                }
#pragma unroll
            for (int r = 0; r < NB; ++r)
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) {
                    if (2 * qs > r) continue;  // compile-time: zero fragment
                    const half8 a = A(ST::s_tb + r * NQS + qs);
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) U[r][ct] = mfma_f16(a, Vb[qs][ct], U[r][ct]);
                }
        }
#pragma unroll
        for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int p = 0; p < KC; ++p) {
                const half8 a = A(ST::s_w + r * KC + p);  // -W
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) UX[r][ct] = mfma_f16(a, XB[p][ct], UX[r][ct]);
            }
#pragma unroll
        for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) U[r][ct][i] = ldexp2(U[r][ct][i], EV - EU) + ldexp2(UX[r][ct][i], E - EU);
        half8 UB[NQS][CTW];
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
                const half4w lo = h4(U[2 * qs][ct]);
                half4w hi = {static_cast<_Float16>(0.f), static_cast<_Float16>(0.f),
                             static_cast<_Float16>(0.f), static_cast<_Float16>(0.f)};
                if (2 * qs + 1 < NB) hi = h4(U[2 * qs + 1 < NB ? 2 * qs + 1 : 0][ct]);
                UB[qs][ct] = cat(lo, hi);
            }

        if constexpr (!SUM) {
            // O^T = qs 2^E X'^T Qt^T + ps 2^EU U'^T P^T per row tile (lane (i, g): token 16r + i,
            // columns col0 + 16ct + 4g .. +3; qs, ps the token row's record multipliers): one
            // 16-byte store per lane and tile; rows past T are beyond the buffer range and dropped
            const float* rowm = reinterpret_cast<const float*>(&L[ST::s_e * 64]);
            const float sc = ldexp2(1.f, E), su = ldexp2(1.f, EU);
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                f32x4 OQ[CTW], OP[CTW];
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) OQ[ct] = OP[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KC; ++p) {
                    const half8 a = A(ST::s_qt + r * KC + p);
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) OQ[ct] = mfma_f16(XB[p][ct], a, OQ[ct]);
                }
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) {
                    if (2 * qs > r) continue;
                    const half8 a = A(ST::s_p + r * NQS + qs);
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) OP[ct] = mfma_f16(UB[qs][ct], a, OP[ct]);
                }
                const float fq = rowm[R.qsc + 16 * r + li] * sc, fp = rowm[R.psc + 16 * r + li] * su;
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Oq[r][ct][i] = fmaf(OP[ct][i], fp, OQ[ct][i] * fq);
            }
        }

        // X' = diag(exp(gam_last)) X + Kb^T U, moved to the domain of U: 2^(E - EU) is folded
        // into the decay factors (0 when X' is zero)
        const float* egl = reinterpret_cast<const float*>(&L[ST::s_e * 64]);
        const int dsh = E - EU;
#pragma unroll
        for (int rt = 0; rt < DKT; ++rt) {
            f32x4 e4 = *reinterpret_cast<const f32x4*>(egl + 16 * rt + 4 * gq);
#pragma unroll
            for (int i = 0; i < 4; ++i) e4[i] = ldexp2(e4[i], dsh);
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) X[rt][ct] *= e4;
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                const half8 a = A(ST::s_kb + rt * NQS + qs);
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) X[rt][ct] = mfma_f16(a, UB[qs][ct], X[rt][ct]);
            }
        }
        E = EU;

        wait_vm();
    };

    if (c1 > c0) {  // a packed sequence with no rows passes its initial state through
        issue_v(VR, c0);
        issue_rec(c0, 0);
        wait_vm();
#pragma nounroll
        for (int n = c0; n < c1; ++n) step(n, (n - c0) & 1);
        store_o(c1 - 1, true);
    }

    float* dst = nullptr;
    if (SUM) dst = xsum + ((size_t)(bh * (NSEG - 1) + seg) * 2 + part) * D * D;
    else if (seg == NSEG - 1 && ht) dst = ht + (size_t)bh * D * D;
    if (dst) {
#pragma unroll
        for (int rt = 0; rt < DKT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(size_t)(16 * rt + 4 * gq + i) * D + col0 + 16 * ct + li] = ldexp2(X[rt][ct][i], E);
    }
}

// Start states of the segments: slot 0 = h0 (or zeros), slot s + 1 = M_s slot s + S_loc_s.
// A workgroup per head and group of CTC 16-column tiles: every workgroup needs all of M_s,
// so with many heads fewer, wider workgroups move fewer bytes per step, and with few heads
// narrow ones spread the sequential walk over more CUs (combine_tiles below).  Wave w owns
// state row tiles 2w and 2w + 1, i.e. exactly the rows of one 32-wide reduction step, which
// it publishes to the other waves as hi/lo fp16 B fragments.  M and S_loc of the
// next segment are requested while the current one is combined.  Range: the start state
// enters the products as S 2^-E (E from its largest magnitude over the workgroup, one extra
// exchange per step), so its hi/lo halves stay inside fp16's range; the transition M is a
// product of non-expansive maps (|M_ij| <= 1 for stable updates) and needs no scale.
template <int D, int CTC>
__global__ __launch_bounds__(2 * D) void carry_combine_kernel(const float* h0, const float* xsum,
                                                           float* sstart, int NH, int NSEG) {
    constexpr int KC = D / 32;
    static_assert((D / 16) % CTC == 0, "column tiles per workgroup");
    __shared__ half8 sB[2][KC][CTC][2][64];
    __shared__ float sMx[2][KC];  // each wave's largest |S|
    const int bh = blockIdx.x % NH;
    const int half = blockIdx.x / NH;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int colb = 16 * CTC * half + li;  // column of tile ct: colb + 16 ct

    auto rowof = [&](int j, int i) { return 16 * (2 * w + j) + 4 * gq + i; };
    f32x4 S[2][CTC];
    float* out0 = sstart + (size_t)bh * NSEG * D * D;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int ct = 0; ct < CTC; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t e = (size_t)rowof(j, i) * D + colb + 16 * ct;
                S[j][ct][i] = h0 ? h0[(size_t)bh * D * D + e] : 0.f;
                out0[e] = S[j][ct][i];
            }

    // operands of one combine step: M rows 16 rt + li (two 4-column pieces per reduction
    // step) and S_loc in accumulator layout
    struct Ops {
        f32x4 m[2][KC][2];
        f32x4 sl[2][CTC];
    };
    auto load_ops = [&](Ops& P, int s) {
        const float* base = xsum + (size_t)(bh * (NSEG - 1) + s) * 2 * D * D;
        const float* M = base + (size_t)D * D;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int rt = 2 * w + j;
#pragma unroll
            for (int p = 0; p < KC; ++p) {
                P.m[j][p][0] = *reinterpret_cast<const f32x4*>(M + (size_t)(16 * rt + li) * D + 32 * p + 4 * gq);
                P.m[j][p][1] = *reinterpret_cast<const f32x4*>(M + (size_t)(16 * rt + li) * D + 32 * p + 16 + 4 * gq);
            }
#pragma unroll
            for (int ct = 0; ct < CTC; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) P.sl[j][ct][i] = base[(size_t)rowof(j, i) * D + colb + 16 * ct];
        }
    };
    Ops cur, nxt;
    if (NSEG > 1) load_ops(cur, 0);
    for (int s = 0; s + 1 < NSEG; ++s) {
        if (s + 2 < NSEG) load_ops(nxt, s + 1);
        const int par = s & 1;
        {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int ct = 0; ct < CTC; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[j][ct][i]));
            m = wave_max(m);
            if (lane == 0) sMx[par][w] = m;
        }
        lds_barrier();
        float mall = sMx[par][0];
#pragma unroll
        for (int ww = 1; ww < KC; ++ww) mall = fmaxf(mall, sMx[par][ww]);
        const int E = mall > 0.f ? exponent_of(mall) - 6 : 0;
        const float sc = ldexp2(1.f, E);
#pragma unroll
        for (int ct = 0; ct < CTC; ++ct) {
            f32x4 s0 = S[0][ct], s1 = S[1][ct];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s0[i] = ldexp2(s0[i], -E);
                s1[i] = ldexp2(s1[i], -E);
            }
            const half4w h0a = h4(s0), h1a = h4(s1);
            f32x4 r0 = s0, r1 = s1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r0[i] -= static_cast<float>(h0a[i]);
                r1[i] -= static_cast<float>(h1a[i]);
            }
            sB[par][w][ct][0][lane] = cat(h0a, h1a);
            sB[par][w][ct][1][lane] = cat(h4(r0), h4(r1));
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f32x4 acc[CTC];
#pragma unroll
            for (int ct = 0; ct < CTC; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < KC; ++p) {
                half8 ah, al;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = cur.m[j][p][hf][i];
                        const _Float16 xh = static_cast<_Float16>(x);
                        ah[4 * hf + i] = xh;
                        al[4 * hf + i] = static_cast<_Float16>(x - static_cast<float>(xh));
                    }
#pragma unroll
                for (int ct = 0; ct < CTC; ++ct) {
                    const half8 bh_ = sB[par][p][ct][0][lane];
                    const half8 bl_ = sB[par][p][ct][1][lane];
                    acc[ct] = mfma_f16(al, bh_, acc[ct]);
                    acc[ct] = mfma_f16(ah, bl_, acc[ct]);
                    acc[ct] = mfma_f16(ah, bh_, acc[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < CTC; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[j][ct][i] = fmaf(acc[ct][i], sc, cur.sl[j][ct][i]);
        }
        float* out = sstart + ((size_t)bh * NSEG + s + 1) * D * D;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int ct = 0; ct < CTC; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) out[(size_t)rowof(j, i) * D + colb + 16 * ct] = S[j][ct][i];
        if (s + 2 < NSEG) cur = nxt;
    }
}

// Column tiles per combine workgroup: the fewest that keep the grid at or below 256
// workgroups (one tile each for up to 32 heads at 128x128; B=1 HV=32 T=32768: 26.5 against
// 38.7 us with two workgroups per head).
inline int combine_tiles(int NH, int D) {
    const int tiles = D / 16;
    int ctc = 1;
    while (ctc < tiles && (long long)NH * (tiles / ctc) > 256) ctc *= 2;
    return ctc;
}

template <typename TIn, int D, int C>
hipError_t launch_wide_t(const LaunchArgs& a, int NC, int NSEG) {
    const int NH = a.B * a.HV;
    hipStream_t st = (hipStream_t)a.stream;
    const unsigned char* ws = (const unsigned char*)a.workspace;
    const CarryLayout L = carry_layout(a.B, a.HV, a.T, a.dk, a.dv, a.chunk, a.plan != nullptr);
    float* xsum = (float*)((unsigned char*)a.workspace + L.xsum_off);
    float* sstart = (float*)((unsigned char*)a.workspace + L.sstart_off);
    if (NSEG > 1) {
        hipLaunchKernelGGL((carry_wide_kernel<TIn, D, C, true>), dim3((unsigned)(NH * (NSEG - 1))), dim3(512),
                           0, st, (const TIn*)a.v, nullptr, nullptr, nullptr, ws, xsum, nullptr, a.B,
                           a.T, a.HV, NC, NSEG, a.plan);
        const int ctc = combine_tiles(NH, D);
        const unsigned nblk = (unsigned)(NH * (D / 16 / ctc));
#define GDR_COMBINE(T_)                                                                        \
    if constexpr ((D / 16) % T_ == 0) {                                                        \
        if (ctc == T_)                                                                         \
            hipLaunchKernelGGL((carry_combine_kernel<D, T_>), dim3(nblk), dim3(2 * D), 0, st,    \
                               a.h0, (const float*)xsum, sstart, NH, NSEG);                    \
    }
        GDR_COMBINE(1) GDR_COMBINE(2) GDR_COMBINE(4) GDR_COMBINE(8)
#undef GDR_COMBINE
    }
    if (a.o_bf16)
        hipLaunchKernelGGL((carry_wide_kernel<TIn, D, C, false, true>), dim3((unsigned)(NH * NSEG)), dim3(256), 0,
                           st, (const TIn*)a.v, a.h0, a.o, a.ht, ws, nullptr, (const float*)sstart, a.B,
                           a.T, a.HV, NC, NSEG, a.plan);
    else
        hipLaunchKernelGGL((carry_wide_kernel<TIn, D, C, false, false>), dim3((unsigned)(NH * NSEG)), dim3(256), 0,
                           st, (const TIn*)a.v, a.h0, a.o, a.ht, ws, nullptr, (const float*)sstart, a.B,
                           a.T, a.HV, NC, NSEG, a.plan);
    return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_wide_d(const LaunchArgs& a, int NC, int NSEG) {
    if (a.chunk == 16) return launch_wide_t<TIn, D, 16>(a, NC, NSEG);
    if (a.chunk == 32) return launch_wide_t<TIn, D, 32>(a, NC, NSEG);
    if (a.chunk == 64) return launch_wide_t<TIn, D, 64>(a, NC, NSEG);
    return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t launch_wide(const LaunchArgs& a, int NC, int NSEG) {
    if (a.dk == 64) return launch_wide_d<TIn, 64>(a, NC, NSEG);
    if (a.dk == 128) return launch_wide_d<TIn, 128>(a, NC, NSEG);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_carry(const LaunchArgs& a) {
    const CarryLayout L = carry_layout(a.B, a.HV, a.T, a.dk, a.dv, a.chunk, a.plan != nullptr);
    if (!L.wide) return launch_carry_split(a);
    const int NC = a.plan ? 0 : (a.T + a.chunk - 1) / a.chunk;  // packed: per sequence
    return a.qkv_f32 ? launch_wide<float>(a, NC, L.nseg) : launch_wide<bf16_t>(a, NC, L.nseg);
}

}  // namespace gdr
