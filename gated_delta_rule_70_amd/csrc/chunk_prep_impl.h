// Chunk-parallel half of the chunkwise WY/UT prefill (gfx950).
//
// ExecuTorch PR #21021 ("Reorder channelwise gated delta rule chunked hot loops for
// autovectorization", second commit summary) evaluates prefill chunk by chunk: per-channel
// log-decay prefixes, the beta-folded triangular transform, WY pseudo-keys and
// pseudo-values, causal query/key terms, then the inter-chunk state carry.  Everything
// except the carry depends on one chunk only, so this kernel runs it for all
// (batch, value head, chunk) triples in parallel and hands the results to the sequential
// carry kernel as fp16 MFMA operand fragments (see ChunkRecord).
//
// For a chunk of C tokens (rows r, s; gam = inclusive prefix of g inside the chunk):
//   gram     A_rs = beta_r sum_c k_rc k_sc exp(gam_rc - gam_sc)   (s < r)
//   causal   P_rs =        sum_c q_rc k_sc exp(gam_rc - gam_sc)   (s <= r)
//   solve    Tinv = (I + A)^-1 by exact 16x16-block forward substitution (the block TRSM
//            of uzu PR #576, "Support TreeUpdateSolve kernel", here on fp32 matrix cores)
//   WY       Tb = Tinv diag(beta);  W = Tb (exp(gam) * K)           (pseudo-keys)
//   carry    Qt = exp(gam) * Q;  Kb = exp(gam_last - gam) * K;  exp(gam_last)
//
// Work split.  One workgroup per chunk, one wave per 16-row block I.  Lane (i, g) of wave
// I (i = lane % 16, g = lane / 16) owns token row 16I + i and, for every 32-channel step
// p, the eight key channels 32p + perm_slot(g, 0..7): exactly the slots of an MFMA
// operand fragment.  So the decay prefix is a 16-lane DPP scan, the carry operands Qt
// are stored straight from registers, and the block's own gram and causal tiles come out
// of its registers.  Accumulator tiles land in "row layout" (lane (i, g) holds row i,
// columns 4g..4g+3), which is again the fragment slot order of the token-reduction
// operands Tb and P.  LDS carries only what crosses waves: block totals of the prefix,
// the key-side operands of the off-diagonal gram blocks, the transposed key tiles of the
// token reductions (W and Kb), and the blocks of Tinv during the solve.
//
// Decay factors (log2 units; every exponential is a hardware exp2).  Inside block I,
//   Z_r = exp(gam_r - gam_m), Zi_r = 1 / Z_r   (m = 16I + 7, the block's middle row)
// for the diagonal tiles, which run on the fp32 matrix cores (16x16x4) so these factors
// keep fp32's range and precision;
// off-diagonal tiles J < I use, in fp16 and with both factors <= 1 while g <= 0,
//   key side   k_s exp(gam_{16J+15} - gam_s)
//   row side   k_r exp(gam_r - gam_{16I-1}) * exp(gam_{16I-1} - gam_{16J+15}).
// Z and Zi stay finite while the decay over 8 consecutive tokens of a block is below ~88
// (mean g above about -11 per token), the range documented in gdr.h.
//
// Query range.  Each wave scales its block's queries by an exact power of two 2^-eq
// (eq = exponent of the block's largest |q|), so the row operands of the off-diagonal
// causal tiles and the P fragments are inside fp16's range for any query magnitude.  Each
// decayed query row Qt_r is formed in fp32 and stored times 2^-er, er = exponent of its own
// largest entry (the decay inside one 16-row block can span more than fp16's range, so
// the scale is per row): each 32-channel step of the row is converted with its own
// exponent, and the steps are then aligned to the row's largest by exact fp16 factors.  The record holds the multipliers 2^er (Qt) and 2^eq (P) of every
// row; the carry applies them to the outputs in fp32.
//
// Fused input prologue (template flags KN, GS): with KN the keys arrive raw and each row is
// used divided by its L2 norm (the lane's row sum of squares, summed over its four lane
// groups); with GS g arrives as gate logits a and the scan takes -softplus(a) directly in
// log2 units.  Everything downstream is unchanged.
//
// Gate heads.  g has HG heads: HG = HV (a gate per value head) or HG = HK (one gate per key
// head, shared by its G = HV / HK value heads); value head h reads gate head h / (HV / HG).
// With a shared gate the unscaled gram sum_c k_rc k_sc exp(gam_rc - gam_sc), the causal
// terms, the decay factors, Qt and Kb are the same for every value head of a group; only
// beta (a row scaling of the gram) and what follows from it differ.  That is the fork of
// the uzu PR #576 review thread on the per-value-head gram: a gram per value head, fused
// with the rest (one workgroup per value head, as for HG = HV), or a gram per key head
// with the solve split off per value head.  Template flag SP builds the second form in one
// kernel: one workgroup per (batch, key head, chunk) computes the shared part once, writes
// it into the records of all G value heads, then runs the solve and W once per value head
// (beta for all of them staged in LDS).  Row-scaling the fp32 gram by beta is the same
// multiplication in both forms, so the two give bitwise the same records.
#pragma once

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// x from lane (row lane - N) of the same 16-lane DPP row, 0 for the first N lanes.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + N, 0xF, 0xF, false));
}

// x from row lane N of the same 16-lane DPP row, in every lane of the row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x150 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// D(16x16) += A(16x4) B(4x16) in fp32.  Lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; D as for the fp16 products.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive input elements of one row, widened to fp32 on use.
template <typename TIn>
struct In4;
template <>
struct In4<bf16_t> {
    uint2 u;
    __device__ __forceinline__ void load(rsrc_t r, int voff) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
        u = uint2{x[0], x[1]};
    }
    __device__ __forceinline__ float operator[](int e) const {
        const uint32_t w = e < 2 ? u.x : u.y;
        return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
};
template <>
struct In4<float> {
    float4 u;
    __device__ __forceinline__ void load(rsrc_t r, int voff) {
        const f32x4 x = buf_load_f32x4(r, voff, 0);
        u = float4{x[0], x[1], x[2], x[3]};
    }
    __device__ __forceinline__ float operator[](int e) const {
        return e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
    }
};

// Largest |q| over a lane's loaded elements.  bf16 magnitudes order like their bit
// patterns with the sign cleared, so the maximum is taken on packed 16-bit integers and
// widened once.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <typename TIn>
struct AbsMax;
template <>
struct AbsMax<bf16_t> {
    u16x2 m = {0, 0};
    __device__ __forceinline__ void add(const In4<bf16_t>& x) {
        const u16x2 a = __builtin_bit_cast(u16x2, x.u.x & 0x7FFF7FFFu);
        const u16x2 b = __builtin_bit_cast(u16x2, x.u.y & 0x7FFF7FFFu);
        m = __builtin_elementwise_max(m, __builtin_elementwise_max(a, b));
    }
    __device__ __forceinline__ float get() const {
        const uint32_t bits = m[0] > m[1] ? m[0] : m[1];
        return __uint_as_float(bits << 16);
    }
};
template <>
struct AbsMax<float> {
    float m = 0.f;
    __device__ __forceinline__ void add(const In4<float>& x) {
        m = fmaxf(m, fmaxf(fmaxf(fabsf(x.u.x), fabsf(x.u.y)), fmaxf(fabsf(x.u.z), fabsf(x.u.w))));
    }
    __device__ __forceinline__ float get() const { return m; }
};

__device__ __forceinline__ float f4(const float4& v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// token index of (channel c, token r) inside a transposed key tile row
template <int C>
__device__ __forceinline__ int kt_swz(int c, int r) {
    if constexpr (C == 64) return r ^ (8 * (c & 7));
    return r;
}

// Fragment of a transposed key tile: row (channel) c, tokens r0 .. r0+3 and r0+16 .. r0+19
// (the second group zero if the chunk has no such tokens).
template <int C, int KTP>
__device__ __forceinline__ half8 kt_frag(const _Float16* tile, int c, int r0) {
    const _Float16* row = tile + c * KTP;
    const uint2 lo = *reinterpret_cast<const uint2*>(row + kt_swz<C>(c, r0));
    const uint2 hi = C > 16 ? *reinterpret_cast<const uint2*>(row + kt_swz<C>(c, r0 + 16)) : uint2{0u, 0u};
    return __builtin_bit_cast(half8, uint4{lo.x, lo.y, hi.x, hi.y});
}

// T_II = (I + A_II)^-1 of one 16x16 unit-lower diagonal block, by forward substitution
// with one row per lane.  `a` holds A_II in row layout (lane (i, g): row i, columns
// 4g .. 4g+3); `at` is a 256-float LDS slot private to the wave; on return tR holds T_II in
// the same row layout.
__device__ __forceinline__ void diag_inverse(float* at, f32x4 a, int li, int gq, float (&tR)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) at[(4 * gq + i) * 16 + li] = a[i];
    asm volatile("" ::: "memory");
    float t[16];
#pragma unroll
    for (int j = 15; j >= 0; --j) {
        float acc = (j == li) ? 1.f : 0.f;
        const float* col = at + j * 16;  // A_II[kk][j] for kk = 0..15
#pragma unroll
        for (int kk = j + 1; kk < 16; ++kk) acc -= t[kk] * col[kk];
        t[j] = acc;
        asm volatile("" : "+v"(t[j])::"memory");  // finish row j before reading the next column
    }
    // T_II back into the same slot, transposed (lane i writes row i), then row layout
    if (gq == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) at[j * 16 + li] = t[j];
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) tR[i] = at[(4 * gq + i) * 16 + li];
}

template <int DK, int C>
struct PrepLds {
    static constexpr int NB = C / 16;
    static constexpr int KC = DK / 32;
    // Transposed key tiles [channel][token], fp16.  At C = 64 a row is exactly 64 tokens and
    // the token index is XOR-swizzled by the channel (multiples of 8, so 4-token groups stay
    // contiguous), which spreads a fragment read's 16 channels over the LDS banks; shorter
    // chunks pad rows instead.
    static constexpr int KTP = C == 64 ? 64 : C + 8;
    static constexpr int TTP = C + 4;  // floats per row of the transposed inverse
    static constexpr int SZ_KT = DK * KTP * 2;
    static constexpr int SZ_AS = (NB > 1 ? NB - 1 : 1) * KC * 1024;
    static constexpr int SZ_TT = C * TTP * 4;
    static constexpr int SZ_U = (SZ_KT + SZ_AS > SZ_TT) ? SZ_KT + SZ_AS : SZ_TT;
    // per block: prefix total, middle-row prefix (DK floats each); then the block's two
    // per-channel decay constants; then its diagonal gram tile (256 floats)
    static constexpr int TMS = 2 * DK > 256 ? 2 * DK : 256;
    // per-(block, channel) off-diagonal decay factors in fp16 (the precision they are
    // applied in), one per off-diagonal tile J <= I - 2
    __host__ __device__ static constexpr int ebase(int I) {
        int b = 0;
        for (int i = 2; i < I; ++i) b += i - 1;
        return b;
    }
    static constexpr int NSE = ebase(NB) > 0 ? ebase(NB) : 1;
};


struct PrepCtx {
    _Float16* sKT;   // (exp(gam) k)^T          [channel][token]  (gram, W)
    _Float16* sKbT;  // (exp(gL - gam) k)^T     [channel][token]  (Kb)         } phase 2-3
    half8* sAs;      // off-diagonal key-side fragments [J][p][lane]           }
    float* sTT;      // Tinv^T                  [token s][token r]             } solve
    float* sTM;      // per block [TMS]: prefix total and middle-row prefix [2][channel], then the
                     // block's decay constants [2][channel], then the diagonal tile,
                     // transposed: A_II, then Tinv_II  [j][k] = X[k][j]
    _Float16* sConE; // off-diagonal decay factors [ebase(I) + I - 2 - J][channel]
    float* sBeta;    // beta per row (0 past the chunk end)
};

// The whole per-chunk computation as seen by wave I (a compile-time block index, so that
// every per-block register array is indexed statically).  All waves pass the same number
// of workgroup barriers.
// SP: the workgroup serves the G value heads h .. h + G - 1 of key head kh, whose records
// are `hstride` bytes apart (the gate is per key head).
template <typename TIn, typename TG, int DK, int C, int I, bool KN, bool GS, bool SP>
__device__ __forceinline__ void prep_wave(const PrepCtx& s, const TIn* __restrict__ q,
                                          const TIn* __restrict__ k, const TG* __restrict__ g,
                                          const float* __restrict__ beta, unsigned char* rec,
                                          long long row0, int T, int HK, int HV, int HG, int h, int kh,
                                          int t0, int L, size_t hstride) {
    constexpr int NB = C / 16;
    constexpr int KC = DK / 32;
    constexpr int DKT = DK / 16;
    constexpr int NQS = (C + 31) / 32;
    constexpr int KTP = PrepLds<DK, C>::KTP;
    constexpr int TMS = PrepLds<DK, C>::TMS;
    constexpr int TTP = PrepLds<DK, C>::TTP;
    constexpr ChunkRecord R = ChunkRecord::make(C, DK);
    constexpr int NT = I / 2 + 1;  // token reduction steps of row tile I

    constexpr int EB = PrepLds<DK, C>::ebase(I);  // this block's first off-diagonal factor
    constexpr int ELT = sizeof(TIn);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int r = 16 * I + li;
    half8* frags = reinterpret_cast<half8*>(rec);
    // Parts shared by the value heads of a group are stored into each of their records.
    const int G = HV / HK;
    const int nw = SP ? G : 1;
    const size_t hs = SP ? hstride / 16 : 0;  // record stride in fragments
    auto put = [&](size_t f, half8 v) {
        for (int j = 0; j < nw; ++j) frags[j * hs + f] = v;
    };

    // ---- 1. loads, g -> log2 units, 16-row inclusive scan ---------------------------------
    // Buffer resources over this sequence's T rows (from row0): a row past the sequence end
    // lies beyond the range and reads as zero, which is exactly the zero padding of the
    // ragged last chunk (g = 0, k = q = 0, beta = 0).  The host keeps every offset below 2^31.
    constexpr int GE = sizeof(TG);  // bytes per g element (fp32 or bf16)
    const int hg = h / (HV / HG);  // gate head
    const rsrc_t rs_g = make_rsrc(g + (size_t)row0 * HG * DK, (uint32_t)T * HG * DK * GE);
    const rsrc_t rs_k = make_rsrc(k + (size_t)row0 * HK * DK, (uint32_t)T * HK * DK * ELT);
    const rsrc_t rs_q = make_rsrc(q + (size_t)row0 * HK * DK, (uint32_t)T * HK * DK * ELT);
    const rsrc_t rs_b = make_rsrc(beta + (size_t)row0 * HV, (uint32_t)T * HV * 4);
    const int tr = t0 + r;  // token row within this batch element
    float x[KC][8];
    In4<TIn> kin[KC][2], qin[KC][2];
    float bta = 0.f;
    if constexpr (!SP) {
        bta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_b, (tr * HV + h) * 4, 0, 0));
    } else if (gq == 0) {  // beta of every value head of the group, staged [head][row]
        for (int j = 0; j < G; ++j)
            s.sBeta[j * C + r] =
                __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_b, (tr * HV + h + j) * 4, 0, 0));
    }
#pragma unroll
    for (int p = 0; p < KC; ++p)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int cb = 32 * p + 16 * hh + 4 * gq;
            f32x4 gv;
            if constexpr (GE == 4) {  // g is read once: streamed, so it does not displace the records
                gv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs_g, ((tr * HG + hg) * DK + cb) * 4, 0, kStream));
            } else {  // four bf16 values, widened exactly (half the bytes; the default policy is faster)
                const auto u = __builtin_amdgcn_raw_buffer_load_b64(rs_g, ((tr * HG + hg) * DK + cb) * 2, 0, 0);
                gv = f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u),
                           __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xFFFF0000u)};
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) x[p][4 * hh + e] = gv[e];
        }
#pragma unroll
    for (int p = 0; p < KC; ++p)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int cb = 32 * p + 16 * hh + 4 * gq;
            kin[p][hh].load(rs_k, ((tr * HK + kh) * DK + cb) * ELT);
            qin[p][hh].load(rs_q, ((tr * HK + kh) * DK + cb) * ELT);
        }
#pragma unroll
    for (int p = 0; p < KC; ++p)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            // rows past the sequence end are padding with no decay (a zero logit would
            // still decay by ln 2)
            float v = GS ? (tr < T ? neg_softplus_log2(x[p][jj]) : 0.f) : x[p][jj] * kLog2e;
            v += row_shr<1>(v);
            v += row_shr<2>(v);
            v += row_shr<4>(v);
            v += row_shr<8>(v);
            x[p][jj] = v;  // local prefix P_r (log2 units) through row r of the block
        }
    if (li == 15 || li == 7) {
        float* dst = s.sTM + I * TMS + (li == 15 ? 0 : DK);
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *reinterpret_cast<float4*>(dst + 32 * p + 16 * hh + 4 * gq) =
                    float4{x[p][4 * hh], x[p][4 * hh + 1], x[p][4 * hh + 2], x[p][4 * hh + 3]};
    }
    if constexpr (!SP) {
        if (gq == 0) s.sBeta[r] = bta;
    }
    lds_barrier();  // B1

    // ---- 2. factors; Qt; transposed key tiles; key-side fragments; diagonal gram ---------
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
    half8 bk[KC], bq[KC];  // row-side operands of the off-diagonal tiles (I > 0)
    float* egl_out = reinterpret_cast<float*>(rec + (size_t)R.nfrag * 1024);
    // Per-channel constants of block I (log2 units; m = middle row, o = gam at the row
    // before the block, gL = gam at the chunk's last row):
    //   slot 0: exp(o + P_m), slot 1: exp(gL - o - P_m), so that exp(gam) and
    //   exp(gL - gam) are the per-element Z = exp(P - P_m) or Zi = exp(P_m - P) times a
    //   constant; factor I - 2 - J: exp(gam_{16I-1} - gam_{16J+15}) for the off-diagonal
    //   tiles J <= I - 2 (the decay over the blocks strictly between J and I), in fp16.
    // One lane per channel computes them; slots 0 and 1 go to this block's sTM slot once
    // no wave reads the totals any more.
    constexpr int NCL = (DK + 63) / 64;  // channels per lane
    float c0[NCL], c1[NCL];
#pragma unroll
    for (int u = 0; u < NCL; ++u) c0[u] = c1[u] = 0.f;
#pragma unroll
    for (int u = 0; u < NCL; ++u) {
        const int c = lane + 64 * u;
        if (c >= DK) break;
        const float md = s.sTM[I * TMS + DK + c];
        float off = 0.f, gl = 0.f;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            const float v = s.sTM[J * TMS + c];
            gl += v;
            if (J < I) off += v;
        }
        c0[u] = ex2(off + md);
        c1[u] = ex2(gl - off - md);
        float between = 0.f;
#pragma unroll
        for (int J = I - 2; J >= 0; --J) {
            between += s.sTM[(J + 1) * TMS + c];
            s.sConE[(EB + I - 2 - J) * DK + c] = static_cast<_Float16>(ex2(between));
        }
        if (I == 0) {  // exp(gam_last), natural base
            const float e = ex2(gl);
            for (int j = 0; j < nw; ++j) egl_out[j * hs * 4 + c] = e;
        }
    }
    // query scale exponent of this block (wave-uniform), from the largest |q| of its rows
    int eq;
    {
        AbsMax<TIn> am;
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) am.add(qin[p][hh]);
        eq = exponent_of(wave_max(am.get()));
    }
    if (gq == 0) {
        const float m = ldexp2(1.f, eq);
        for (int j = 0; j < nw; ++j) egl_out[j * hs * 4 + R.psc + 16 * I + li] = m;
    }
    // with raw keys, this row's 1 / |k|_2 (its dk entries sit in lanes li + 16g)
    float rn = 1.f;
    if constexpr (KN) {
        float s2 = 0.f;
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) s2 = fmaf(kin[p][hh][e], kin[p][hh][e], s2);
        rn = inv_key_norm(sum_over_groups(s2));
    }
    // Every wave is past reading the other blocks' totals once this barrier is passed, so a
    // wave may reuse its own block's slot: first for its decay constants, after this phase
    // for its diagonal tile.  Only this wave reads the slot from here on, and a wave's LDS
    // accesses complete in issue order.
    lds_barrier();  // B1b
    float* con = s.sTM + I * TMS;
#pragma unroll
    for (int u = 0; u < NCL; ++u) {
        const int c = lane + 64 * u;
        if (c >= DK) break;
        con[c] = c0[u];
        con[DK + c] = c1[u];
    }
    asm volatile("" ::: "memory");
    half8 qh[KC];  // decayed query row, per 32-channel step times 2^-ep[p]
    int ep[KC];
#pragma unroll
    for (int p = 0; p < KC; ++p) {
        asm volatile("" ::: "memory");  // keep this step's LDS reads here (register pressure)
        // middle-row prefix and block total of each channel: rows 7 and 15 of the lane's
        // 16-lane row, which holds one token row per lane for the same channels
        half8 as;
        float qe[8];
        float pm = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int cb = 32 * p + 16 * hh + 4 * gq;
            const float4 k2 = *reinterpret_cast<const float4*>(con + cb);
            const float4 k3 = *reinterpret_cast<const float4*>(con + DK + cb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 4 * hh + e;
                const int c = cb + e;
                const float kv = KN ? kin[p][hh][e] * rn : kin[p][hh][e];
                const float qv = qin[p][hh][e];
                // middle-row prefix and block total of this channel: rows 7 and 15 of the
                // lane's 16-lane row, which holds one token row per lane for the same channels
                const float dz = x[p][jj] - row_bcast<7>(x[p][jj]);
                const float z = ex2(dz);
                const float zi = ex2(-dz);
                const float eg = z * f4(k2, e);
                qe[jj] = qv * eg;
                pm = fmaxf(pm, fabsf(qe[jj]));
                s.sKT[c * KTP + kt_swz<C>(c, r)] = static_cast<_Float16>(kv * eg);
                s.sKbT[c * KTP + kt_swz<C>(c, r)] = static_cast<_Float16>(kv * (zi * f4(k3, e)));
                // diagonal tiles on the fp32 matrix cores: reduction step = this slot's channel
                // in each of the four lane groups
                const float a = kv * zi;
                accA = mfma_f32(a, kv * z, accA);
                accP = mfma_f32(a, qv * z, accP);
                if constexpr (I > 0) {
                    const float zs = ex2(x[p][jj]);  // exp(gam - gam_{16I-1}) <= 1
                    bk[p][jj] = static_cast<_Float16>(kv * zs);
                    bq[p][jj] = static_cast<_Float16>(ldexp2(qv * zs, -eq));
                }
                if constexpr (I < NB - 1)
                    as[jj] = static_cast<_Float16>(kv * ex2(row_bcast<15>(x[p][jj]) - x[p][jj]));
            }
        }
        if constexpr (I < NB - 1) s.sAs[(I * KC + p) * 64 + lane] = as;
        ep[p] = exponent_of(max_over_groups(pm));  // row r's entries of this step: lanes li + 16g
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) qh[p][jj] = static_cast<_Float16>(ldexp2(qe[jj], -ep[p]));
    }
    {  // Qt row r times 2^-er, er = the row's largest step exponent
        int er = ep[0];
#pragma unroll
        for (int p = 1; p < KC; ++p) er = max(er, ep[p]);
#pragma unroll
        for (int p = 0; p < KC; ++p) {
            const _Float16 f = half_pow2(ep[p] - er);
            put((size_t)(R.off_qt + I * KC + p) * 64 + lane, qh[p] * half8{f, f, f, f, f, f, f, f});
        }
        if (gq == 0) {
            const float m = ldexp2(1.f, er);
            for (int j = 0; j < nw; ++j) egl_out[j * hs * 4 + R.qsc + 16 * I + li] = m;
        }
    }
    // diagonal tiles in row layout: gram rows times beta_r (per value head with SP),
    // strictly lower; causal lower
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * gq + i;
        accA[i] = sl < li ? (SP ? accA[i] : accA[i] * bta) : 0.f;
        accP[i] = sl <= li ? ldexp2(accP[i], -eq) : 0.f;
    }

    // ---- diagonal block inverse, rows by lane: T_II = (I + A_II)^-1 ----------------------
    // Only this wave's rows are involved (its own sTM slot: the decay constants there are
    // dead once phase 2 is over), so without SP it runs while the other waves finish phase 2.
    float* at = s.sTM + I * TMS;
    float tR[4];
    if constexpr (!SP) diag_inverse(at, accA, li, gq, tR);
    lds_barrier();  // B2

    // ---- 3. off-diagonal gram tiles; Kb and P fragments ---------------------------------
    // aR[J], pR[J]: rows of block I against the columns of block J, in row layout.
    f32x4 aR[I + 1], pR[I + 1];
    aR[I] = accA;
    pR[I] = accP;
#pragma unroll
    for (int J = 0; J < I; ++J) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, pc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KC; ++p) {
            half8 ak = s.sAs[(J * KC + p) * 64 + lane];
            if (J < I - 1) {
                // blocks between J and I: scale the key side by exp(gam_{16I-1} - gam_{16J+15})
                const _Float16* er = s.sConE + (EB + I - 2 - J) * DK + 32 * p + 4 * gq;
                const uint2 e0 = *reinterpret_cast<const uint2*>(er);
                const uint2 e1 = *reinterpret_cast<const uint2*>(er + 16);
                ak = ak * __builtin_bit_cast(half8, uint4{e0.x, e0.y, e1.x, e1.y});
            }
            a = mfma_f16(ak, bk[p], a);
            pc = mfma_f16(ak, bq[p], pc);
        }
        aR[J] = a;
        pR[J] = pc;
    }
#pragma unroll
    for (int f = I; f < DKT * NQS; f += NB) {
        const int ct = f / NQS, qs = f % NQS;
        put((size_t)(R.off_kb + f) * 64 + lane, kt_frag<C, KTP>(s.sKbT, 16 * ct + li, 32 * qs + 4 * gq));
    }
    if constexpr (!SP) {
#pragma unroll
        for (int J = 0; J < I; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) aR[J][i] *= bta;
    }
#pragma unroll
    for (int qs = 0; qs < NT; ++qs) {  // fragments above the diagonal are zero and never read
        half8 v;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int J = 2 * qs + (jj >> 2);
            v[jj] = J <= I ? static_cast<_Float16>(pR[J <= I ? J : I][jj & 3]) : static_cast<_Float16>(0.f);
        }
        put((size_t)(R.off_p + I * NQS + qs) * 64 + lane, v);
    }
    lds_barrier();  // B3: the key-side fragments and the Kb tile are dead; solve area live

    // Phases 4 and 5 for one value head: its beta per row (sb), the lane's own row beta as
    // the gram's row scale (bsc, SP only: without SP the gram is already scaled) and its
    // record (fr).
    auto solve = [&](const float* sb, float bsc, half8* fr) {
    // ---- 4. publish T_II into Tinv^T ------------------------------------------------------
#pragma unroll
    for (int i = 0; i < 4; ++i) s.sTT[(16 * I + 4 * gq + i) * TTP + 16 * I + li] = tR[i];
    lds_barrier();  // B4

    // ---- 5. off-diagonal inverse blocks, one block row per stage ------------------------
    //   T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ; stage d finishes block row d.  Products run on
    //   the fp32 matrix cores: the row-layout A_IM is the A operand and column-layout T_MJ
    //   (lane (j, g) holds T_MJ[4g .. 4g+3][j], read from Tinv^T) the B operand, with
    //   reduction index 4g + kk in step kk, so accumulators come out in column layout.
    f32x4 Y[I > 0 ? I : 1];
#pragma unroll
    for (int J = 0; J < I; ++J) Y[J] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Tb fragments and pseudo-keys of block row I, once that row of Tinv is final
    auto finish_row = [&]() {
        half8 tb[NT];
#pragma unroll
        for (int qs = 0; qs < NT; ++qs) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int J = 2 * qs + hh;
                if (J > I) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) tb[qs][4 * hh + i] = static_cast<_Float16>(0.f);
                } else {
                    const float4 b4 = *reinterpret_cast<const float4*>(sb + 16 * J + 4 * gq);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float tv = (J == I) ? tR[i] : s.sTT[(16 * J + 4 * gq + i) * TTP + 16 * I + li];
                        tb[qs][4 * hh + i] = static_cast<_Float16>(tv * f4(b4, i));
                    }
                }
            }
            fr[(size_t)(R.off_tb + I * NQS + qs) * 64 + lane] = tb[qs];
        }

        // W^T = (exp(gam) K)^T Tb^T: A operand from the transposed key tile, B operand Tb
#pragma unroll
        for (int p = 0; p < KC; ++p) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qs = 0; qs < NT; ++qs) {
                const half8 k0 = kt_frag<C, KTP>(s.sKT, 32 * p + li, 32 * qs + 4 * gq);
                const half8 k1 = kt_frag<C, KTP>(s.sKT, 32 * p + 16 + li, 32 * qs + 4 * gq);
                a0 = mfma_f16(k0, tb[qs], a0);
                a1 = mfma_f16(k1, tb[qs], a1);
            }
            half8 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[i] = static_cast<_Float16>(-a0[i]);
                w[4 + i] = static_cast<_Float16>(-a1[i]);
            }
            fr[(size_t)(R.off_w + I * KC + p) * 64 + lane] = w;
        }
    };

#pragma unroll
    for (int d = 1; d < NB; ++d) {
        if (I >= d) {
            const int M = d - 1;
#pragma unroll
            for (int J = 0; J <= M; ++J) {
                const f32x4 tm = *reinterpret_cast<const f32x4*>(s.sTT + (16 * J + li) * TTP + 16 * M + 4 * gq);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) Y[J] = mfma_f32(SP ? aR[M][kk] * bsc : aR[M][kk], tm[kk], Y[J]);
            }
            if (I == d) {
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) z = mfma_f32(tR[kk], Y[J][kk], z);
                    *reinterpret_cast<f32x4*>(s.sTT + (16 * J + li) * TTP + 16 * I + 4 * gq) = -z;
                }
                asm volatile("" ::: "memory");
            }
        }
        if (I == d - 1) finish_row();
        if (d < NB - 1) lds_barrier();
    }
    if constexpr (I == NB - 1) finish_row();
    };

    if constexpr (!SP) {
        solve(s.sBeta, 1.f, frags);
    } else {
        for (int j = 0; j < G; ++j) {
            // the previous head's solve has finished reading the solve area everywhere
            if (j > 0) lds_barrier();
            const float* sb = s.sBeta + j * C;
            const float bj = sb[r];
            f32x4 ad;
#pragma unroll
            for (int i = 0; i < 4; ++i) ad[i] = accA[i] * bj;
            diag_inverse(at, ad, li, gq, tR);
            solve(sb, bj, frags + j * hs);
        }
    }
}


// Three workgroups per CU (LDS and the 168-register budget allow it); the raw-key variant
// and the split form need a few more registers and run two per CU rather than spill.
template <typename TIn, typename TG, int DK, int C, bool KN, bool GS, bool SP>
__global__ __launch_bounds__(C * 4, (KN || SP) ? 2 : 3) void chunk_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TG* __restrict__ g,
    const float* __restrict__ beta, unsigned char* __restrict__ ws, int B, int T, int HK, int HV,
    int HG, int NC, const int32_t* __restrict__ plan) {
    using Lds = PrepLds<DK, C>;
    constexpr int NB = C / 16;
    constexpr ChunkRecord R = ChunkRecord::make(C, DK);
    __shared__ __align__(16) _Float16 sKT[DK * Lds::KTP];
    __shared__ __align__(16) float sTM[NB * Lds::TMS];
    __shared__ __align__(16) _Float16 sConE[Lds::NSE * DK];
    __shared__ __align__(16) float sBeta[SP ? kSplitMaxGroup * C : C];  // [value head][row] with SP
    __shared__ __align__(16) unsigned char sU[Lds::SZ_U];
    PrepCtx s;
    s.sKT = sKT;
    s.sKbT = reinterpret_cast<_Float16*>(sU);
    s.sAs = reinterpret_cast<half8*>(sU + Lds::SZ_KT);
    s.sTT = reinterpret_cast<float*>(sU);
    s.sTM = sTM;
    s.sConE = sConE;
    s.sBeta = sBeta;

    // Items are (batch element, key head, chunk) triples, chunk fastest -- or, for a packed
    // variable-length batch (plan != nullptr), (key head, chunk slot) pairs, the slot's
    // sequence read from the plan; NC is then the number of chunk slots.
    const int G = HV / HK;
    const int blk = blockIdx.x;
    const long long items = plan ? (long long)HK * NC : (long long)B * HK * NC;
    int pair, sub;
    if constexpr (SP) {
        // one item per block, serving value heads kh*G .. kh*G+G-1
        pair = blk;
        sub = 0;
    } else {
        // Block -> item: the G value heads that share a key head (and so read the same q and
        // k rows) get blocks 8 apart, i.e. the same XCD (blocks are dealt round-robin to the
        // 8 XCDs) at about the same time, so all but the first read of each q/k row hit that
        // XCD's L2.  Runs of 8G blocks cover 8 items; the last run's unused blocks return
        // at once.
        const int within = blk % (8 * G);
        pair = (blk / (8 * G)) * 8 + within % 8;
        sub = within / 8;
    }
    if (pair >= items) return;
    int b, kh, n;
    SeqSpan sp;
    if (plan) {
        const int slot = pair % NC;
        if (slot >= plan[VarlenPlan::first(B) + B]) return;  // past the last sequence's chunks
        kh = pair / NC;
        b = plan[VarlenPlan::chunk_seq(B) + slot];
        sp = seq_span(plan, b, B, T, NC);
        n = slot - sp.c0;
    } else {
        n = pair % NC;
        kh = (pair / NC) % HK;
        b = pair / NC / HK;
        sp = seq_span(nullptr, b, B, T, NC);
    }
    const int h = kh * G + sub;
    const int t0 = n * C;
    const int L = min(C, sp.T - t0);
    const size_t hstride = (size_t)sp.nc * R.bytes;  // between the records of heads h and h + 1
    unsigned char* rec = ws + ((size_t)sp.c0 * HV + (size_t)h * sp.nc + n) * R.bytes;
    const int I = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#define GDR_WAVE(I_)                                                                            \
    if (I == I_) {                                                                              \
        if constexpr (I_ < NB)                                                                  \
            prep_wave<TIn, TG, DK, C, I_, KN, GS, SP>(s, q, k, g, beta, rec, sp.row0, sp.T, HK, HV, \
                                                      HG, h, kh, t0, L, hstride);               \
        return;                                                                                 \
    }
    GDR_WAVE(0) GDR_WAVE(1) GDR_WAVE(2) GDR_WAVE(3)
#undef GDR_WAVE
}

// Launch of the prep kernel for one instantiation: blocks as the kernel maps them.
template <typename TIn, typename TG, int DK, int C, bool KN, bool GS, bool SP>
hipError_t launch_prep_t(const LaunchArgs& a) {
    // dense: chunks per batch element; packed: chunk slots
    const int NC = a.plan ? a.nct : (a.T + C - 1) / C;
    const long long items = (long long)(a.plan ? 1 : a.B) * a.HK * NC;
    const long long blocks = SP ? items : (items + 7) / 8 * 8 * (a.HV / a.HK);
    hipLaunchKernelGGL((chunk_prep_kernel<TIn, TG, DK, C, KN, GS, SP>), dim3((unsigned)blocks), dim3(C * 4), 0,
                       (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TG*)a.g, a.beta,
                       (unsigned char*)a.workspace, a.B, a.T, a.HK, a.HV, a.HG, NC, a.plan);
    return hipGetLastError();
}

// Every (dk, chunk, input type, prologue) instantiation of one form.
template <typename TIn, typename TG, bool KN, bool GS, bool SP>
hipError_t dispatch_prep(const LaunchArgs& a) {
#define GDR_CASE(DK_, C_) \
    if (a.dk == DK_ && a.chunk == C_) return launch_prep_t<TIn, TG, DK_, C_, KN, GS, SP>(a);
    GDR_CASE(32, 16) GDR_CASE(32, 32) GDR_CASE(32, 64)
    GDR_CASE(64, 16) GDR_CASE(64, 32) GDR_CASE(64, 64)
    GDR_CASE(128, 16) GDR_CASE(128, 32) GDR_CASE(128, 64)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

template <bool KN, bool GS, bool SP>
hipError_t dispatch_prep_types(const LaunchArgs& a) {
    if (a.qkv_f32) return dispatch_prep<float, float, KN, GS, SP>(a);
    return a.g_bf16 ? dispatch_prep<bf16_t, bf16_t, KN, GS, SP>(a) : dispatch_prep<bf16_t, float, KN, GS, SP>(a);
}

template <bool SP>
hipError_t dispatch_prep_form(const LaunchArgs& a) {
    if (a.k_l2norm)
        return a.g_softplus ? dispatch_prep_types<true, true, SP>(a) : dispatch_prep_types<true, false, SP>(a);
    return a.g_softplus ? dispatch_prep_types<false, true, SP>(a) : dispatch_prep_types<false, false, SP>(a);
}

}  // namespace
}  // namespace gdr
