// Sequential half of the chunkwise WY/UT prefill: the inter-chunk state carry (gfx950).
//
// With the chunk operands prepared by chunk_prep (decayed queries Qt, pseudo-keys W,
// decay-to-end keys Kb, Tb = (I + A)^-1 diag(beta), causal terms P, exp(gam_last)), one
// chunk advances the state S (dk x dv) as
//   U    = Tb V - W S                  pseudo-values minus the state's prediction
//   O    = Qt S + P U                  outputs of the chunk's tokens
//   S'   = diag(exp(gam_last)) S + Kb^T U
// (ExecuTorch PR #21021 "Reorder channelwise gated delta rule chunked hot loops for
// autovectorization", second commit summary: WY pseudo-keys/values and inter-chunk state
// carry).  Columns of S evolve independently, so the value dimension is split across
// workgroups: a workgroup owns NT 16-column tiles of one (batch, value head) and walks
// the chunks in order.
//
// Inside a workgroup the chunk's rows are split across NW = C/16 waves: wave w computes
// row tile w of U and O and owns the state row tiles ct = w, w + NW, ...  Per chunk the
// waves exchange two small fp16 operand sets through LDS (the state's B fragments, then
// U's), one barrier each, so the chain U -> S' that bounds the recurrence runs on all
// SIMDs of a CU and each wave loads only the share of the chunk's operands it uses.
// Every product is a 16x16x32 fp16 MFMA with fp32 accumulation; accumulator tiles map
// to B fragments without shuffles (reduction slots follow perm_slot).
//
// Memory pipeline: each wave keeps its operand fragments and the raw v rows in a ring of
// three register sets.  At the start of chunk n it requests chunk n+2's operands into the
// set chunk n-1 has just released (buffer loads, fragment index in an SGPR), so every
// load has two whole chunks of work to land; outputs are stored one chunk late.  The
// chunk step is straight-line code (no per-wave branches), which keeps the compiler's
// memory-wait counts at the pipeline's real depth.
//
// Range.  The state and v enter the products as fp16, each in its own scaled domain: per
// chunk each wave scales its state tiles by 2^-es_w and its v rows by 2^-ev_w (exponents of
// their largest magnitudes) before publishing them with the exponents; a reader takes
// E_S = max_w es_w, E_V = max_w ev_w and aligns every fragment half to them with exact fp16
// power-of-two factors.  Tb V and W S go to separate accumulators and meet in fp32 at the
// larger scale E_U = max(E_S, E_V), so a state far smaller than v (or the reverse) keeps its
// precision; U is published at 2^-E_U, the state update adds 2^E_U Kb^T U, and the outputs
// are 2^E_S Qt S + 2^E_U P U with the query rows' record multipliers (see chunk_prep).  So
// every product stays inside fp16's range for state and v magnitudes within fp32's normal
// range; U itself keeps fp16's precision while beta >= 2^-12 (or beta = 0 exactly).
//
// Launch: blocks = (B*HV) x (dv / (16*NT)), block index = colgroup * (B*HV) + head, so
// all column groups of a head share one XCD (blocks are dealt round-robin to the 8 XCDs)
// and read the head's records through one L2.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// x from lane j (0..15) of the same 16-lane DPP row, in every lane of the row; j must fold
// to a constant.
__device__ __forceinline__ float row_lane(float x, int j) {
#define GDR_BC(J) \
    case J: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + J, 0xF, 0xF, false));
    switch (j) {
        GDR_BC(0) GDR_BC(1) GDR_BC(2) GDR_BC(3) GDR_BC(4) GDR_BC(5) GDR_BC(6) GDR_BC(7)
        GDR_BC(8) GDR_BC(9) GDR_BC(10) GDR_BC(11) GDR_BC(12) GDR_BC(13) GDR_BC(14)
        default: GDR_BC(15)
    }
#undef GDR_BC
}

__device__ __forceinline__ half4 to_half4(f32x4 x) {
    return half4{static_cast<_Float16>(x[0]), static_cast<_Float16>(x[1]), static_cast<_Float16>(x[2]),
                 static_cast<_Float16>(x[3])};
}
// x * 2^e, then fp16
__device__ __forceinline__ half4 to_half4_scaled(f32x4 x, int e) {
    return half4{static_cast<_Float16>(ldexp2(x[0], e)), static_cast<_Float16>(ldexp2(x[1], e)),
                 static_cast<_Float16>(ldexp2(x[2], e)), static_cast<_Float16>(ldexp2(x[3], e))};
}

// Scale exponents of the carry's fp16 operands: a published block of values with largest
// magnitude m is stored times 2^-(exponent(m) - kTgt), i.e. with its maximum in [32, 64);
// U = Tb V - W S then stays below 64 (|Tb|_1 + |W|_1) < 65504 for any well-conditioned
// chunk.  kNoExp marks an all-zero block (it never sets the common exponent).
constexpr int kTgt = 6;
constexpr int kNoExp = -1000;
__device__ __forceinline__ int scale_exponent(float m) { return m > 0.f ? exponent_of(m) - kTgt : kNoExp; }

// Largest |x| over the raw bits of v held by a lane (bf16 pairs or fp32).
template <typename TIn>
__device__ __forceinline__ float raw_absmax(uint32_t x) {
    if constexpr (sizeof(TIn) == 2) {
        const uint32_t a = x & 0x7FFF7FFFu;  // bf16 magnitudes order like their bits
        const uint32_t hi = a >> 16, lo = a & 0xFFFFu;
        return __uint_as_float((hi > lo ? hi : lo) << 16);
    } else {
        return fabsf(__uint_as_float(x));
    }
}

template <typename TIn, int DK, int DV, int C, int NT, bool OBF>
__global__ __launch_bounds__(64 * (C / 16)) void chunk_carry_kernel(
    const TIn* __restrict__ v, const float* h0, void* __restrict__ o, float* ht,
    const unsigned char* __restrict__ ws, int B, int T, int HV, int NC, const int32_t* __restrict__ plan) {
    constexpr int obf = OBF;  // o stored as bf16 (a compile-time choice: no branch per store)
    constexpr int NB = C / 16;
    constexpr int NW = NB;                    // one wave per 16-row tile of the chunk
    constexpr int NQS = (C + 31) / 32;
    constexpr int KC = DK / 32;
    constexpr int DKT = DK / 16;
    constexpr int OWN = (DKT + NW - 1) / NW;  // state row tiles per wave (at most)
    constexpr ChunkRecord R = ChunkRecord::make(C, DK);
    constexpr int ELT = sizeof(TIn);

    // exchange buffers, three copies (chunk index mod 3), lane-major: state B fragments
    // [KC][NT], U B fragments [NQS][NT]; and the chunk's v tile [nt][col][row] in fp16,
    // columns padded to VP halves so the 16 columns a fragment read touches fall in
    // different LDS banks
    constexpr int VP = C + 4;
    __shared__ half8 sSB[3][KC * NT * 64];
    __shared__ half8 sUB[3][NQS * NT * 64];
    __shared__ __attribute__((aligned(16))) _Float16 sV[3][NT * 16 * VP];
    __shared__ int sE[3][8];  // each wave's state and v scale exponents, per exchange copy

    const int NH = B * HV;
    const int blk = blockIdx.x;
    const int bh = blk % NH;
    const int cg = blk / NH;
    const int h = bh % HV;
    const int b = bh / HV;
    // this batch element's (or packed sequence's) rows, chunks and first chunk slot
    const SeqSpan sp = seq_span(plan, b, B, T, NC);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // row tile of this wave
    __builtin_assume(w >= 0 && w < NW);  // lets the compiler drop the per-tile guards
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;

    int jcol[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) jcol[nt] = 16 * (cg * NT + nt) + li;

    // owned state tiles in accumulator layout: S[j][nt][i] = S[16 ct_j + 4gq + i][jcol[nt]]
    f32x4 S[OWN][NT];
    const size_t sb = (size_t)bh * DK * DV;
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
        const int ct = w + NW * j;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (h0 != nullptr && ct < DKT) {  // uniform
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = h0[sb + (size_t)(16 * ct + 4 * gq + i) * DV + jcol[nt]];
            }
            S[j][nt] = x;
        }
    }

    // Buffer resources: this head's records, and this batch element's v and o rows (the
    // host guarantees each fits a 31-bit byte offset).  Wave-uniform offsets (fragment
    // index, row within a chunk) go to SGPRs; one per-lane offset is built per chunk.
    const unsigned char* rec0 = ws + ((size_t)sp.c0 * HV + (size_t)h * sp.nc) * R.bytes;
    const int rowv = HV * DV * ELT;  // bytes between consecutive tokens of v
    const int rowo = HV * DV * o_elt(obf);  // ... of o
    const rsrc_t rs_rec = make_rsrc(rec0, (uint32_t)sp.nc * R.bytes);
    const rsrc_t rs_v = make_rsrc(v + (size_t)sp.row0 * HV * DV, (uint32_t)sp.T * rowv);
    const rsrc_t rs_o =
        make_rsrc(static_cast<unsigned char*>(o) + (size_t)sp.row0 * rowo, (uint32_t)sp.T * rowo);

    // v rows of a chunk.  Wave w loads rows 16w .. 16w+15 of its workgroup's 16*NT columns
    // with one vector load per 16-column tile (lane l: row l/4, four columns 4(l%4)..),
    // keeping the raw bits in registers until the chunk starts; rows past T sit beyond the
    // buffer's range (the row is part of the per-lane offset) and read as zero.  At the
    // start of the chunk the rows go to a column-major fp16 tile in LDS, from which every
    // wave reads the B fragments of Tb V (reduction slots follow perm_slot).
    typedef uint32_t VRaw[NT][ELT];  // 4 elements of one row per lane and column tile
    auto load_v = [&](int n, VRaw& V) {
        const int row = n * C + 16 * w + (lane >> 2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int off = (row * HV + h) * DV * ELT + (16 * (cg * NT + nt) + 4 * (lane & 3)) * ELT;
            if constexpr (ELT == 2) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs_v, off, 0, 0);
                V[nt][0] = x[0];
                V[nt][1] = x[1];
            } else {
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs_v, off, 0, 0);
                V[nt][0] = x[0];
                V[nt][1] = x[1];
                V[nt][2] = x[2];
                V[nt][3] = x[3];
            }
        }
    };
    auto publish_v = [&](const VRaw& V, _Float16* dst, int ew) {  // -> [nt][col][row], fp16 * 2^-ew
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x;
                if constexpr (ELT == 2) x = __uint_as_float((e & 1) ? (V[nt][e >> 1] & 0xFFFF0000u) : (V[nt][e >> 1] << 16));
                else x = __uint_as_float(V[nt][e]);
                dst[(nt * 16 + 4 * (lane & 3) + e) * VP + 16 * w + (lane >> 2)] = static_cast<_Float16>(ldexp2(x, -ew));
            }
    };
    auto read_v = [&](half8 (&V)[NQS][NT], const _Float16* src) {
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const _Float16* col = &src[(nt * 16 + li) * VP + 32 * qs + 4 * gq];
                const half4 lo = *reinterpret_cast<const half4*>(col);
                half4 hi = {static_cast<_Float16>(0.f), static_cast<_Float16>(0.f),
                            static_cast<_Float16>(0.f), static_cast<_Float16>(0.f)};
                if (32 * qs + 16 < C) hi = *reinterpret_cast<const half4*>(col + 16);  // compile-time
                V[qs][nt] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    };
    // outputs of row tile w of chunk n, held transposed (lane (i, g): row 16w + i, columns
    // 4g .. 4g+3 of each column tile), so one 16-byte store per lane and tile; rows past T
    // fall outside the buffer and are dropped (the row stays in the per-lane offset so one
    // form serves every chunk)
    auto store_o = [&](int n, const f32x4 (&O)[NT]) {
        const int obase = ((n * C + 16 * w + li) * HV + h) * DV * 4 + (16 * cg * NT + 4 * gq) * 4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) store_o4_stream(O[nt], rs_o, obase, nt * 64, obf);
    };

    // This wave's operand fragments, in registers, in a ring of three sets (the empty asm
    // keeps a load where it is written; the compiler would otherwise sink it to its next
    // use and stall).  The chunk loop is unrolled by three so each set has fixed registers.
    struct Frags {
        half8 tb[NQS], w[KC], q[KC], p[NQS], kb[OWN][NQS];
        f32x4 e;                 // exp(gam_last) of owned state tile j, in row lane j
        float qs, ps;            // Qt and P row multipliers of this lane's token row
        uint32_t v[NT][ELT];     // raw bits of this wave's v rows of the chunk
    };
    // A per-lane offset past every record range: such a load reads zeros without touching
    // memory (the range check applies to the per-lane offset, not to the SGPR one).
    constexpr int kBeyond = (int)0xFFFFFF00u;
    auto ld = [&](half8& dst, int vrec, int f) {
        dst = buf_load_half8(rs_rec, vrec, f * 1024);
        asm volatile("" ::: "memory");
    };
    // exp(gam_last) of the owned state tiles, one load per wave: row lane j of lane group g
    // reads rows 16 ct_j + 4g .. +3 (the other lanes read zeros from beyond the range); the
    // values are broadcast along the row at use time
    auto ld_egl = [&](int n) {
        const int ct = w + NW * li;
        const bool on = li < OWN && ct < DKT;
        return buf_load_f32x4(rs_rec, on ? n * R.bytes + ct * 64 + gq * 16 : kBeyond, R.nfrag * 1024);
    };
    // A chunk's operands are requested in four groups spread over the step two chunks
    // earlier, so the vector-memory unit works through them while the step computes
    // instead of holding up the wave behind a burst of requests.
    auto ld_g1 = [&](Frags& F, int n) {  // v rows, Tb, P
        const int vrec = n * R.bytes + lane * 16;
        load_v(n, F.v);
        // Tb and P fragments above row tile w's diagonal are zero: read them from beyond the
        // range instead of from memory (a per-wave choice of offset, no branch)
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            const int vq = 2 * qs > w ? kBeyond : vrec;
            ld(F.tb[qs], vq, R.off_tb + w * NQS + qs);
            ld(F.p[qs], vq, R.off_p + w * NQS + qs);
        }
    };
    auto ld_g2 = [&](Frags& F, int n) {  // W
        const int vrec = n * R.bytes + lane * 16;
#pragma unroll
        for (int p = 0; p < KC; ++p) ld(F.w[p], vrec, R.off_w + w * KC + p);
    };
    auto ld_g3 = [&](Frags& F, int n) {  // Qt
        const int vrec = n * R.bytes + lane * 16;
#pragma unroll
        for (int p = 0; p < KC; ++p) ld(F.q[p], vrec, R.off_qt + w * KC + p);
    };
    auto ld_g4 = [&](Frags& F, int n) {  // Kb, exp(gam_last)
        const int vrec = n * R.bytes + lane * 16;
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) ld(F.kb[j][qs], vrec, R.off_kb + ct * NQS + qs);
            }
        }
        F.e = ld_egl(n);
        const int rs = n * R.bytes + (16 * w + li) * 4;  // token row 16w + li of the chunk
        F.qs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_rec, rs, R.nfrag * 1024 + R.qsc * 4, 0));
        F.ps = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_rec, rs, R.nfrag * 1024 + R.psc * 4, 0));
    };
    auto load_all = [&](Frags& F, int n) {
        ld_g1(F, n);
        ld_g2(F, n);
        ld_g3(F, n);
        ld_g4(F, n);
    };

    f32x4 Op[NT];  // outputs of the previous chunk (true scale), stored one step late

    // This wave's scale exponents for the next chunk step: largest magnitudes of its state
    // tiles and of that chunk's v rows.  Each step computes them for the following one right
    // after its state update, where the reductions overlap the step's output products rather
    // than delay the next step's first exchange.
    int es, ev;
    auto state_exponent = [&]() {
        float ms = 0.f;
#pragma unroll
        for (int j = 0; j < OWN; ++j)
            if (w + NW * j < DKT)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[j][nt][i]));
        return scale_exponent(wave_max(ms));
    };
    auto v_exponent = [&](const Frags& F) {
        float mv = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < ELT; ++e) mv = fmaxf(mv, raw_absmax<TIn>(F.v[nt][e]));
        return scale_exponent(wave_max(mv));
    };

    // One chunk: request chunk nn's operands into set Fn, consume set F (chunk n), using
    // exchange-buffer copy `par`; Fx holds the next chunk's operands.
    auto step = [&](Frags& F, Frags& Fn, Frags& Fx, int n, int nn, int par) {
        ld_g1(Fn, nn);
        // The empty asm fixes where the raw v bits are consumed: the compiler would otherwise
        // convert them a step early, while their load may still be in flight.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < ELT; ++e) asm volatile("" : "+v"(F.v[nt][e]));

        publish_v(F.v, sV[par], ev);

        // 1. publish this wave's state tiles (times 2^-es) as halves of the state B fragments
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    *(reinterpret_cast<half4*>(&sSB[par][((ct >> 1) * NT + nt) * 64 + lane]) + (ct & 1)) =
                        to_half4_scaled(S[j][nt], -es);
            }
        }
        if (lane == 0) {
            sE[par][w] = es;
            sE[par][4 + w] = ev;
        }
        lds_barrier();
        // common exponents and the factors 2^(e_w - E) that align each wave's halves to them
        int esw[NW], evw[NW];
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            esw[ww] = sE[par][ww];
            evw[ww] = sE[par][4 + ww];
        }
        int ES = esw[0], EV = evw[0];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
            ES = max(ES, esw[ww]);
            EV = max(EV, evw[ww]);
        }
        const int EU = max(ES, EV);
        _Float16 fs[NW], fv[NW];
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            fs[ww] = half_pow2(esw[ww] - ES);
            fv[ww] = half_pow2(evw[ww] - EV);
        }
        // a B fragment of reduction step p holds row tiles 2p and 2p+1 (owners (2p) % NW and
        // (2p+1) % NW), a v fragment of token step qs rows 16(2qs) .. 16(2qs+2) (waves 2qs, 2qs+1)
        auto align = [&](half8 x, const _Float16 (&f)[NW], int wa, int wb) {
            const _Float16 a = f[wa % NW], b = f[wb % NW];
            return x * half8{a, a, a, a, b, b, b, b};
        };
        half8 SB[KC][NT];
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) SB[p][nt] = align(sSB[par][(p * NT + nt) * 64 + lane], fs, 2 * p, 2 * p + 1);
        half8 Vc[NQS][NT];
        read_v(Vc, sV[par]);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Vc[qs][nt] = align(Vc[qs][nt], fv, 2 * qs, 2 * qs + 1 < NW ? 2 * qs + 1 : 2 * qs);
        // the scaled domains back to true scale

        if (n > 0) store_o(n - 1, Op);
        ld_g2(Fn, nn);

        // 2. U_w = Tb V - W S for row tile w (times 2^-E_U; the two products meet in fp32)
        f32x4 U[NT], US[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) U[nt] = US[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) U[nt] = mfma_f16(F.tb[qs], Vc[qs][nt], U[nt]);
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) US[nt] = mfma_f16(F.w[p], SB[p][nt], US[nt]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) U[nt][i] = ldexp2(U[nt][i], EV - EU) + ldexp2(US[nt][i], ES - EU);
        // 3. publish U_w as half of a U B fragment
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *(reinterpret_cast<half4*>(&sUB[par][((w >> 1) * NT + nt) * 64 + lane]) + (w & 1)) = to_half4(U[nt]);
        ld_g3(Fn, nn);
        // 4. O_w^T = S^T Qt^T (independent of U; overlaps the exchange).  The operands swap
        // places: a fragment reads the same as an A operand of X and a B operand of X^T.
        f32x4 OQ[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) OQ[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) OQ[nt] = mfma_f16(SB[p][nt], F.q[p], OQ[nt]);
        lds_barrier();
        half8 UB[NQS][NT];
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                half8 x = sUB[par][(qs * NT + nt) * 64 + lane];
                if (2 * qs + 1 >= NB) {  // compile-time: this step has no second row tile
#pragma unroll
                    for (int jj = 4; jj < 8; ++jj) x[jj] = static_cast<_Float16>(0.f);
                }
                UB[qs][nt] = x;
            }
        ld_g4(Fn, nn);

        // 5. S' = diag(exp(gam_last)) S + 2^E_U Kb^T U for the owned state tiles
        const float su = ldexp2(1.f, EU);
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
                f32x4 ej;
#pragma unroll
                for (int i = 0; i < 4; ++i) ej[i] = row_lane(F.e[i], j);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int qs = 0; qs < NQS; ++qs) a = mfma_f16(F.kb[j][qs], UB[qs][nt], a);
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[j][nt][i] = fmaf(a[i], su, S[j][nt][i] * ej[i]);
                }
            }
        }
        // 0'. the next step's exponents (Fx's v loads were issued a step earlier)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < ELT; ++e) asm volatile("" : "+v"(Fx.v[nt][e]));
        es = state_exponent();
        ev = v_exponent(Fx);
        // 6. O_w^T = qs 2^E_S S^T Qt^T + ps 2^E_U U^T P^T, the query rows' multipliers per lane
        const float fq = F.qs * ldexp2(1.f, ES), fp = F.ps * su;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 OP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) OP = mfma_f16(UB[qs][nt], F.p[qs], OP);
#pragma unroll
            for (int i = 0; i < 4; ++i) Op[nt][i] = fmaf(OP[i], fp, OQ[nt][i] * fq);
        }
    };

    // A sequence with no rows (packed batches) passes its initial state through.
    const int nc = sp.nc;
    if (nc > 0) {
        Frags FA, FB, FC;
        load_all(FA, 0);
        load_all(FB, min(1, nc - 1));
        es = state_exponent();
        ev = v_exponent(FA);
        // Three steps per iteration (register set and exchange copy fixed per position), then
        // up to two more; the requested chunk is clamped to the last one, whose operands then
        // simply arrive twice.
        int n = 0;
        for (; n + 3 <= nc; n += 3) {
            step(FA, FC, FB, n, min(n + 2, nc - 1), 0);
            step(FB, FA, FC, n + 1, min(n + 3, nc - 1), 1);
            step(FC, FB, FA, n + 2, min(n + 4, nc - 1), 2);
        }
        if (n < nc) step(FA, FC, FB, n, min(n + 2, nc - 1), 0);
        if (n + 1 < nc) step(FB, FA, FC, n + 1, min(n + 3, nc - 1), 1);
        store_o(nc - 1, Op);
    }

    if (ht) {
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ht[sb + (size_t)(16 * ct + 4 * gq + i) * DV + jcol[nt]] = S[j][nt][i];
            }
        }
    }
}

// The same chunk step for one 16-column tile per workgroup, split over two wave roles
// (2 * C/16 waves, two per SIMD).  Chain waves (row tile w) carry the state: they publish S,
// form U_w = Tb_w V - W_w S, publish U_w and update their state tiles
// S' = diag(exp(gam_last)) S + Kb^T U, then take the next step's state exponent.  Output
// waves (row tile w) load, scale and publish the chunk's v rows with their exponent before
// the first barrier, and form the outputs from the two exchanges: O_w^T = S^T Qt_w^T after
// the first barrier and + U^T P_w^T after the second.  The v stream, the output operands,
// products and stores thus stay out of the chain waves' instruction stream and vector-memory
// counter.  Each role keeps its own ring of three operand sets, loaded two chunks ahead as
// above, and spreads the loads of one set over the step: the chain waves issue Tb after the
// first barrier (not ahead of the state publish), the output waves issue P after it, and a
// chunk's outputs are stored one step late, after the next chunk's first barrier, so no
// store sits in the queue ahead of the loads a step waits for.  B=1 T=4097, HV=32, 128x128,
// the carry right after the prep kernel: 70.5 us against 80 with every load of a set issued
// at the top of the step and the stores at its end, and 82 for the one-role kernel, all
// bitwise the same results.
template <typename TIn, int DK, int DV, int C, bool OBF>
__global__ __launch_bounds__(128 * (C / 16)) void chunk_carry_roles_kernel(
    const TIn* __restrict__ v, const float* h0, void* __restrict__ o, float* ht,
    const unsigned char* __restrict__ ws, int B, int T, int HV, int NC, const int32_t* __restrict__ plan) {
    constexpr int obf = OBF;  // o stored as bf16 (a compile-time choice: no branch per store)
    constexpr int NT = 1;
    constexpr int NB = C / 16;
    constexpr int NW = NB;
    constexpr int NQS = (C + 31) / 32;
    constexpr int KC = DK / 32;
    constexpr int DKT = DK / 16;
    constexpr int OWN = (DKT + NW - 1) / NW;
    constexpr ChunkRecord R = ChunkRecord::make(C, DK);
    constexpr int ELT = sizeof(TIn);
    constexpr int VP = C + 4;
    // exchange buffers as in chunk_carry_kernel (three copies, chunk index mod 3): the chain
    // waves write the state fragments, U and the state exponents, the output waves v and
    // its exponents
    __shared__ half8 sSB[3][KC * 64];
    __shared__ half8 sUB[3][NQS * 64];
    __shared__ __attribute__((aligned(16))) _Float16 sV[3][16 * VP];
    __shared__ int sE[3][8];

    const int NH = B * HV;
    const int blk = blockIdx.x;
    const int bh = blk % NH;
    const int cg = blk / NH;
    const int h = bh % HV;
    const int b = bh / HV;
    const SeqSpan sp = seq_span(plan, b, B, T, NC);
    const int nc = sp.nc;
    // waves 0 .. NW-1 carry the state, NW .. 2NW-1 form the outputs; both own row tile w
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool outw = wv >= NW;
    const int w = outw ? wv - NW : wv;  // row tile
    __builtin_assume(w >= 0 && w < NW);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int jcol = 16 * cg + li;
    const unsigned char* rec0 = ws + ((size_t)sp.c0 * HV + (size_t)h * sp.nc) * R.bytes;
    const rsrc_t rs_rec = make_rsrc(rec0, (uint32_t)sp.nc * R.bytes);
    constexpr int kBeyond = (int)0xFFFFFF00u;
    auto ld = [&](half8& dst, int vrec, int f) {
        dst = buf_load_half8(rs_rec, vrec, f * 1024);
        asm volatile("" ::: "memory");
    };
    // common exponents of exchange copy `par` and the factors that align each wave's halves
    struct Exps {
        int ES, EV, EU;
        _Float16 fs[NW], fv[NW];
    };
    auto read_exps = [&](int par) {
        Exps x;
        int esw[NW], evw[NW];
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            esw[ww] = sE[par][ww];
            evw[ww] = sE[par][4 + ww];
        }
        x.ES = esw[0];
        x.EV = evw[0];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
            x.ES = max(x.ES, esw[ww]);
            x.EV = max(x.EV, evw[ww]);
        }
        x.EU = max(x.ES, x.EV);
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            x.fs[ww] = half_pow2(esw[ww] - x.ES);
            x.fv[ww] = half_pow2(evw[ww] - x.EV);
        }
        return x;
    };
    auto align = [&](half8 x, const _Float16 (&f)[NW], int wa, int wb) {
        const _Float16 a = f[wa % NW], bb = f[wb % NW];
        return x * half8{a, a, a, a, bb, bb, bb, bb};
    };
    auto read_sb = [&](half8 (&SB)[KC], int par, const Exps& x) {
#pragma unroll
        for (int p = 0; p < KC; ++p) SB[p] = align(sSB[par][p * 64 + lane], x.fs, 2 * p, 2 * p + 1);
    };
    auto read_ub = [&](half8 (&UB)[NQS], int par) {
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            half8 x = sUB[par][qs * 64 + lane];
            if (2 * qs + 1 >= NB) {
#pragma unroll
                for (int jj = 4; jj < 8; ++jj) x[jj] = static_cast<_Float16>(0.f);
            }
            UB[qs] = x;
        }
    };

    const int rowv = HV * DV * ELT;
    const rsrc_t rs_v = make_rsrc(v + (size_t)sp.row0 * HV * DV, (uint32_t)sp.T * rowv);
    typedef uint32_t VRaw[ELT];
    auto load_v = [&](int n, VRaw& V) {
        const int row = n * C + 16 * w + (lane >> 2);
        const int off = (row * HV + h) * DV * ELT + (16 * cg + 4 * (lane & 3)) * ELT;
        if constexpr (ELT == 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs_v, off, 0, 0);
            V[0] = x[0];
            V[1] = x[1];
        } else {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs_v, off, 0, 0);
            V[0] = x[0];
            V[1] = x[1];
            V[2] = x[2];
            V[3] = x[3];
        }
    };
    auto publish_v = [&](const VRaw& V, _Float16* dst, int ew) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x;
            if constexpr (ELT == 2) x = __uint_as_float((e & 1) ? (V[e >> 1] & 0xFFFF0000u) : (V[e >> 1] << 16));
            else x = __uint_as_float(V[e]);
            dst[(4 * (lane & 3) + e) * VP + 16 * w + (lane >> 2)] = static_cast<_Float16>(ldexp2(x, -ew));
        }
    };
    auto read_v = [&](half8 (&V)[NQS], const _Float16* src) {
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            const _Float16* col = &src[li * VP + 32 * qs + 4 * gq];
            const half4 lo = *reinterpret_cast<const half4*>(col);
            half4 hi = {static_cast<_Float16>(0.f), static_cast<_Float16>(0.f), static_cast<_Float16>(0.f),
                        static_cast<_Float16>(0.f)};
            if (32 * qs + 16 < C) hi = *reinterpret_cast<const half4*>(col + 16);
            V[qs] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // Both roles pass the same barriers: B0, then B1(n) and B2(n) for every chunk n.
    if (outw) {
        // ---- output waves: v rows, Qt and P fragments of row tile w and the row multipliers,
        // two chunks ahead; each chunk's outputs stored during the next chunk's step ----
        const int rowo = HV * DV * o_elt(obf);
        const rsrc_t rs_o =
            make_rsrc(static_cast<unsigned char*>(o) + (size_t)sp.row0 * rowo, (uint32_t)sp.T * rowo);
        struct OFr {
            half8 q[KC], p[NQS];
            float qs, ps;
            uint32_t v[ELT];
        };
        auto load_ov = [&](OFr& F, int n) {
            load_v(n, F.v);
            asm volatile("" ::: "memory");
        };
        auto load_oq = [&](OFr& F, int n) {
            const int vrec = n * R.bytes + lane * 16;
#pragma unroll
            for (int p = 0; p < KC; ++p) ld(F.q[p], vrec, R.off_qt + w * KC + p);
            const int rs = n * R.bytes + (16 * w + li) * 4;
            F.qs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_rec, rs, R.nfrag * 1024 + R.qsc * 4, 0));
        };
        auto load_op = [&](OFr& F, int n) {
            const int vrec = n * R.bytes + lane * 16;
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) ld(F.p[qs], 2 * qs > w ? kBeyond : vrec, R.off_p + w * NQS + qs);
            const int rs = n * R.bytes + (16 * w + li) * 4;
            F.ps = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_rec, rs, R.nfrag * 1024 + R.psc * 4, 0));
        };
        auto load_o = [&](OFr& F, int n) {
            load_ov(F, n);
            load_op(F, n);
            load_oq(F, n);
        };
        f32x4 Opend = {0.f, 0.f, 0.f, 0.f};  // the previous chunk's outputs and their offset
        int opend = -1;
        auto ostep = [&](OFr& F, OFr& Fn, int n, int nn, int par) {
            load_ov(Fn, nn);
            load_oq(Fn, nn);
#pragma unroll
            for (int e = 0; e < ELT; ++e) asm volatile("" : "+v"(F.v[e]));
            {  // this row tile's v rows of chunk n, times 2^-ev, and their exponent
                float mv = 0.f;
#pragma unroll
                for (int e = 0; e < ELT; ++e) mv = fmaxf(mv, raw_absmax<TIn>(F.v[e]));
                const int evn = scale_exponent(wave_max(mv));
                publish_v(F.v, sV[par], evn);
                if (lane == 0) sE[par][4 + w] = evn;
            }
            lds_barrier();  // B1(n)
            if (opend >= 0) store_o4_stream(Opend, rs_o, opend, 0, obf);
            load_op(Fn, nn);
            const Exps x = read_exps(par);
            half8 SB[KC];
            read_sb(SB, par, x);
            f32x4 OQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < KC; ++p) OQ = mfma_f16(SB[p], F.q[p], OQ);
            lds_barrier();  // B2(n)
            half8 UB[NQS];
            read_ub(UB, par);
            f32x4 OP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) OP = mfma_f16(UB[qs], F.p[qs], OP);
            const float fq = F.qs * ldexp2(1.f, x.ES), fp = F.ps * ldexp2(1.f, x.EU);
            f32x4 Ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) Ov[i] = fmaf(OP[i], fp, OQ[i] * fq);
            const int obase = ((n * C + 16 * w + li) * HV + h) * DV * 4 + (16 * cg + 4 * gq) * 4;
            Opend = Ov;
            opend = obase;
        };
        lds_barrier();  // B0
        if (nc > 0) {
            OFr FA, FB, FC;
            load_o(FA, 0);
            load_o(FB, min(1, nc - 1));
            int n = 0;
            for (; n + 3 <= nc; n += 3) {
                ostep(FA, FC, n, min(n + 2, nc - 1), 0);
                ostep(FB, FA, n + 1, min(n + 3, nc - 1), 1);
                ostep(FC, FB, n + 2, min(n + 4, nc - 1), 2);
            }
            if (n < nc) ostep(FA, FC, n, min(n + 2, nc - 1), 0);
            if (n + 1 < nc) ostep(FB, FA, n + 1, min(n + 3, nc - 1), 1);
            store_o4_stream(Opend, rs_o, opend, 0, obf);
        }
        return;
    }

    // ---- chain waves: the state tiles and the Tb, W, Kb fragments of row tile w ----
    f32x4 S[OWN];
    const size_t sb = (size_t)bh * DK * DV;
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
        const int ct = w + NW * j;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (h0 != nullptr && ct < DKT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = h0[sb + (size_t)(16 * ct + 4 * gq + i) * DV + jcol];
        }
        S[j] = x;
    }
    struct Frags {
        half8 tb[NQS], w[KC], kb[OWN][NQS];
        f32x4 e;
    };
    auto ld_egl = [&](int n) {
        const int ct = w + NW * li;
        const bool on = li < OWN && ct < DKT;
        return buf_load_f32x4(rs_rec, on ? n * R.bytes + ct * 64 + gq * 16 : kBeyond, R.nfrag * 1024);
    };
    auto ld_g1 = [&](Frags& F, int n) {
        const int vrec = n * R.bytes + lane * 16;
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) ld(F.tb[qs], 2 * qs > w ? kBeyond : vrec, R.off_tb + w * NQS + qs);
    };
    auto ld_g2 = [&](Frags& F, int n) {
        const int vrec = n * R.bytes + lane * 16;
#pragma unroll
        for (int p = 0; p < KC; ++p) ld(F.w[p], vrec, R.off_w + w * KC + p);
    };
    auto ld_g4 = [&](Frags& F, int n) {
        const int vrec = n * R.bytes + lane * 16;
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) ld(F.kb[j][qs], vrec, R.off_kb + ct * NQS + qs);
            }
        }
        F.e = ld_egl(n);
    };
    auto load_all = [&](Frags& F, int n) {
        ld_g1(F, n);
        ld_g2(F, n);
        ld_g4(F, n);
    };
    int es;
    auto state_exponent = [&]() {
        float ms = 0.f;
#pragma unroll
        for (int j = 0; j < OWN; ++j)
            if (w + NW * j < DKT)
#pragma unroll
                for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[j][i]));
        return scale_exponent(wave_max(ms));
    };
    auto step = [&](Frags& F, Frags& Fn, Frags& Fx, int n, int nn, int par) {
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT)
                *(reinterpret_cast<half4*>(&sSB[par][(ct >> 1) * 64 + lane]) + (ct & 1)) = to_half4_scaled(S[j], -es);
        }
        if (lane == 0) sE[par][w] = es;
        lds_barrier();  // B1(n)
        ld_g1(Fn, nn);
        const Exps x = read_exps(par);
        half8 SB[KC];
        read_sb(SB, par, x);
        half8 Vc[NQS];
        read_v(Vc, sV[par]);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) Vc[qs] = align(Vc[qs], x.fv, 2 * qs, 2 * qs + 1 < NW ? 2 * qs + 1 : 2 * qs);
        ld_g2(Fn, nn);
        f32x4 U = {0.f, 0.f, 0.f, 0.f}, US = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) U = mfma_f16(F.tb[qs], Vc[qs], U);
#pragma unroll
        for (int p = 0; p < KC; ++p) US = mfma_f16(F.w[p], SB[p], US);
#pragma unroll
        for (int i = 0; i < 4; ++i) U[i] = ldexp2(U[i], x.EV - x.EU) + ldexp2(US[i], x.ES - x.EU);
        *(reinterpret_cast<half4*>(&sUB[par][(w >> 1) * 64 + lane]) + (w & 1)) = to_half4(U);
        lds_barrier();  // B2(n)
        half8 UB[NQS];
        read_ub(UB, par);
        ld_g4(Fn, nn);
        const float su = ldexp2(1.f, x.EU);
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
                f32x4 ej;
#pragma unroll
                for (int i = 0; i < 4; ++i) ej[i] = row_lane(F.e[i], j);
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) a = mfma_f16(F.kb[j][qs], UB[qs], a);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[j][i] = fmaf(a[i], su, S[j][i] * ej[i]);
            }
        }
        es = state_exponent();
    };
    lds_barrier();  // B0
    if (nc > 0) {
        Frags FA, FB, FC;
        load_all(FA, 0);
        load_all(FB, min(1, nc - 1));
        es = state_exponent();
        int n = 0;
        for (; n + 3 <= nc; n += 3) {
            step(FA, FC, FB, n, min(n + 2, nc - 1), 0);
            step(FB, FA, FC, n + 1, min(n + 3, nc - 1), 1);
            step(FC, FB, FA, n + 2, min(n + 4, nc - 1), 2);
        }
        if (n < nc) step(FA, FC, FB, n, min(n + 2, nc - 1), 0);
        if (n + 1 < nc) step(FB, FA, FC, n + 1, min(n + 3, nc - 1), 1);
    }
    if (ht) {
#pragma unroll
        for (int j = 0; j < OWN; ++j) {
            const int ct = w + NW * j;
            if (ct < DKT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) ht[sb + (size_t)(16 * ct + 4 * gq + i) * DV + jcol] = S[j][i];
            }
        }
    }
}

template <typename TIn, int DK, int DV, int C, bool OBF>
static hipError_t launch_carry_roles_o(const LaunchArgs& a) {
    const int NC = a.plan ? 0 : (a.T + C - 1) / C;
    const long long nblk = (long long)a.B * a.HV * (DV / 16);
    hipLaunchKernelGGL((chunk_carry_roles_kernel<TIn, DK, DV, C, OBF>), dim3((unsigned)nblk), dim3(128 * (C / 16)),
                       0, (hipStream_t)a.stream, (const TIn*)a.v, a.h0, a.o, a.ht, (const unsigned char*)a.workspace,
                       a.B, a.T, a.HV, NC, a.plan);
    return hipGetLastError();
}
template <typename TIn, int DK, int DV, int C>
static hipError_t launch_carry_roles(const LaunchArgs& a) {
    return a.o_bf16 ? launch_carry_roles_o<TIn, DK, DV, C, true>(a) : launch_carry_roles_o<TIn, DK, DV, C, false>(a);
}

template <typename TIn, int DK, int DV, int C, int NT, bool OBF>
static hipError_t launch_carry_o(const LaunchArgs& a) {
    const int NC = a.plan ? 0 : (a.T + C - 1) / C;  // packed batches: per sequence, from the plan
    const long long nblk = (long long)a.B * a.HV * (DV / (16 * NT));
    hipLaunchKernelGGL((chunk_carry_kernel<TIn, DK, DV, C, NT, OBF>), dim3((unsigned)nblk),
                       dim3(64 * (C / 16)), 0, (hipStream_t)a.stream, (const TIn*)a.v, a.h0, a.o,
                       a.ht, (const unsigned char*)a.workspace, a.B, a.T, a.HV, NC, a.plan);
    return hipGetLastError();
}
template <typename TIn, int DK, int DV, int C, int NT>
static hipError_t launch_carry_t(const LaunchArgs& a) {
    return a.o_bf16 ? launch_carry_o<TIn, DK, DV, C, NT, true>(a) : launch_carry_o<TIn, DK, DV, C, NT, false>(a);
}

// Column split: with few heads every 16-column tile gets its own workgroup (the most
// parallel carry, for B*HV too small to fill 256 CUs otherwise; the two-role kernel); with
// many heads a workgroup covers several tiles so each head's records are read from L2 fewer
// times.
template <typename TIn, int DK, int DV, int C>
static hipError_t dispatch_split(const LaunchArgs& a) {
    constexpr int CT = DV / 16;
    const long long tiles = (long long)a.B * a.HV * CT;
    // the fewest tiles per workgroup that keep the grid within one round of 256 workgroups
    // (B = 4 T = 1024, HV = 32, 128 x 128: 59 us with 4 tiles against 108 with one, which
    // needs four rounds)
    if constexpr (CT >= 4 && C >= 32) {
        if (tiles > 512) return launch_carry_t<TIn, DK, DV, C, 4>(a);
    }
    if constexpr (CT >= 2) {
        if (tiles > 256) return launch_carry_t<TIn, DK, DV, C, 2>(a);
    }
    return launch_carry_roles<TIn, DK, DV, C>(a);
}

template <typename TIn, int DK, int DV>
static hipError_t dispatch_chunk(const LaunchArgs& a) {
    if (a.chunk == 16) return dispatch_split<TIn, DK, DV, 16>(a);
    if (a.chunk == 32) return dispatch_split<TIn, DK, DV, 32>(a);
    if (a.chunk == 64) return dispatch_split<TIn, DK, DV, 64>(a);
    return hipErrorInvalidValue;
}

template <typename TIn>
static hipError_t dispatch_carry(const LaunchArgs& a) {
#define GDR_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return dispatch_chunk<TIn, DK_, DV_>(a);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_carry_split(const LaunchArgs& a) {
    return a.qkv_f32 ? dispatch_carry<float>(a) : dispatch_carry<bf16_t>(a);
}

}  // namespace gdr
