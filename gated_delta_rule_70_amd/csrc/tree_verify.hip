// Tree-verify solve of the channelwise gated delta rule, gfx950.
//
// uzu PR #576 ("Support TreeUpdateSolve kernel") verifies a speculative token tree with a
// gram over the tree's tokens, a kh0 term (keys times the initial state) and an exact
// block triangular solve.  Here every node of a tree of T <= 64 tokens continues the
// recurrence from its parent's state (the parent of node t is parent[t] < t, -1 for the
// initial state h0) and its output is that of the plain recurrence along its root path.
// Unrolled along a path, that is the chunk algebra of one chunk with the causal order
// replaced by ancestry:
//   gam_t  = g_t + gam_parent(t)                   (decay prefix along the root path)
//   A_rs   = beta_r sum_c k_rc k_sc exp(gam_rc - gam_sc)   for s a strict ancestor of r
//   P_rs   =        sum_c q_rc k_sc exp(gam_rc - gam_sc)   for s = r or an ancestor of r
//   U      = (I + A)^-1 diag(beta) (V - (exp(gam) k) h0)  (forward substitution)
//   O      = (exp(gam) q) h0 + P U
// A and P are dot products of Kt = exp(gam) k (or Qt = exp(gam) q) with
// Kh = exp(-gam) k; every term that survives the ancestry mask is bounded by 1, the
// masked ones are finite while the path decay stays above -80 in every channel.
//
// One 256-thread workgroup per (batch, value head, group of 32-column blocks of v), all of
// a tree's rows in LDS; with enough heads a group holds 2 or 4 blocks, which share the
// decayed rows, A, P and the diagonal inverses (phases 1, 3 and the inversion of 4 run once
// per group, phases 2, 4 and 5 once per block; B=8 T=64 at 128x128: 28 against 63 us with
// one block per workgroup, bitwise the same outputs).  Every phase is parallel across nodes:
//   0. all global reads issued at once (parents, beta, g, k, q rows, the block's columns
//      of h0 and v);
//   1. ancestor masks by pointer doubling in one wave's registers (6 rounds cover any depth
//      below 64), root-path decay prefixes as one 0/1-matrix product on the fp32 matrix
//      cores (whatever the depth), then the decayed rows, kept as bf16 high/low pairs;
//   2. Kt h0 and Qt h0 (three bf16 matrix-core products per tile on the split operands,
//      fp32 accumulation), the right-hand side;
//   3. A and P the same way, masked by ancestry;
//   4. (I + A) U = rhs by 16-row blocks: each diagonal block (unit lower triangular, since
//      node order is a topological order) is inverted in registers by forward substitution
//      down its columns, then block I takes U_I = inv(D_I) (rhs_I - sum_{J<I} A_IJ U_J) on
//      the matrix cores; the serial depth is the number of blocks, whatever the tree's depth;
//   5. O = Qt h0 + P U on the fp32 matrix cores.
// The solve and everything after it run in fp32; the split products of phases 2 and 3 keep
// each product within ~3 * 2^-16 of the fp32 one.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {
namespace {

constexpr int TM = 64;  // most nodes per tree
constexpr int CB = 32;  // v columns per workgroup

// D(16x16) += A(16x4) B(4x16) in fp32.  Lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; D rows 4g .. 4g+3 of column l % 16 (g = l / 16).
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split of four fp32 values into bf16 high parts and bf16 remainders (round to nearest even
// on both): x = hi + lo to 2^-16 relative.  Pairs are converted together and the high
// parts widened back by shifting their bits (x - hi is exact: hi is x's nearest bf16).
__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const f32x2 v = {x[2 * h], x[2 * h + 1]};
        const bf16x2 hb = __builtin_convertvector(v, bf16x2);
        const uint32_t u = __builtin_bit_cast(uint32_t, hb);
        const f32x2 hf = {__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u)};
        const bf16x2 lb = __builtin_convertvector(v - hf, bf16x2);
        hi[2 * h] = hb[0];
        hi[2 * h + 1] = hb[1];
        lo[2 * h] = lb[0];
        lo[2 * h + 1] = lb[1];
    }
}

// sum over a K-long reduction of X[rowA][.] * Y[rowB][.] for a 16x16 tile, both operands
// held as bf16 high/low pairs (each low part `xlo` / `ylo` elements after its high part),
// as three bf16 matrix-core products hi*hi + hi*lo + lo*hi with fp32 accumulation: the
// split and the dropped lo*lo term leave each product within ~3 * 2^-16 of the exact one.
// Lane (i, g) reads 8 consecutive slots at 32 s + 8 g of row i of X and of Y (xa, yb point
// at slot 8 g); D rows 4g .. 4g+3 of column i.  Every operand read is issued first.
template <int K>
__device__ __forceinline__ f32x4 tile_dot_split(const __bf16* xa, int xlo, const __bf16* yb, int ylo) {
    constexpr int NS = K / 32;
    bf16x8 xh[NS], xl[NS], yh[NS], yl[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        xh[st] = *reinterpret_cast<const bf16x8*>(xa + 32 * st);
        yh[st] = *reinterpret_cast<const bf16x8*>(yb + 32 * st);
        xl[st] = *reinterpret_cast<const bf16x8*>(xa + xlo + 32 * st);
        yl[st] = *reinterpret_cast<const bf16x8*>(yb + ylo + 32 * st);
    }
    f32x4 hh = {0.f, 0.f, 0.f, 0.f}, hl = hh, lh = hh;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        hh = mfma_bf16(xh[st], yh[st], hh);
        hl = mfma_bf16(xh[st], yl[st], hl);
        lh = mfma_bf16(xl[st], yh[st], lh);
    }
    return hh + (hl + lh);
}

// acc + X[16 rows][0 .. 4L) Y[0 .. 4L)[16 columns] for one 16x16 tile in fp32 (16x16x4
// products), lane group g taking the contiguous reduction range gL .. gL + L - 1: xa points
// at element gL of row i (16-byte aligned), yb at row gL of column i, Y's rows ys apart.
// Every read is issued before the products.
template <int L>
__device__ __forceinline__ f32x4 tile_rows_cols(const float* xa, const float* yb, int ys, f32x4 acc) {
    f32x4 xv[L / 4];
    float yv[L];
#pragma unroll
    for (int i = 0; i < L / 4; ++i) xv[i] = *reinterpret_cast<const f32x4*>(xa + 4 * i);
#pragma unroll
    for (int k = 0; k < L; ++k) yv[k] = yb[k * ys];
#pragma unroll
    for (int k = 0; k < L; ++k) acc = mfma4(xv[k / 4][k % 4], yv[k], acc);
    return acc;
}

// One 16x16 tile of M Y for a 0/1 matrix M given by bit masks: lane group g reduces over
// L consecutive rows of Y, bit k of `bits` (the lane's row of M shifted to the group's
// first column) selecting row k; yb points at the group's first row of column i, rows ys
// apart.  Every read is issued before the products; the sums are plain fp32 sums.
template <int L>
__device__ __forceinline__ f32x4 prefix_tile(unsigned long long bits, const float* yb, int ys) {
    float yv[L];
#pragma unroll
    for (int k = 0; k < L; ++k) yv[k] = yb[k * ys];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < L; ++k) acc = mfma4((bits >> k) & 1ull ? 1.f : 0.f, yv[k], acc);
    return acc;
}

// KN: keys given raw (each row used divided by its L2 norm); GS: g given as gate logits
// (log-decay -softplus(a)).  The fused input prologue, applied where the rows are loaded.
template <typename TIn, typename TG, int DK, bool KN, bool GS>
__global__ __launch_bounds__(256) void tree_verify_kernel(
    const int32_t* __restrict__ parent, const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const TG* __restrict__ g, const float* __restrict__ beta,
    const float* __restrict__ h0, void* __restrict__ o, int T, int HK, int HV, int HG, int DV, int ncbw,
    int obf) {
    constexpr int KP = DK + 4;   // row pitch (floats) of the fp32 g rows and decay prefixes
    constexpr int AP = TM + 4;
    constexpr int UP = CB + 4;
    constexpr int BP = DK + 8;   // bf16 row pitch: 16-byte reads of 16 rows hit distinct banks
    constexpr int ELT = sizeof(TIn);
    constexpr int LO = TM * BP;  // offset of the low parts in a split row array
    static_assert(2 * CB * BP * 2 <= TM * AP * 4 && CB * (TM + 4) <= TM * AP,
                  "staging must fit A and P");
    static_assert(TM * KP * 4 <= 2 * TM * BP * 2, "g rows and prefixes must fit a split row array");
    // decayed rows as bf16 high parts [TM][BP] followed by low parts [TM][BP]
    __shared__ __attribute__((aligned(16))) __bf16 sKt[2 * TM * BP];  // exp(gam) k
    __shared__ __attribute__((aligned(16))) __bf16 sKh[2 * TM * BP];  // exp(-gam) k
    __shared__ __attribute__((aligned(16))) __bf16 sQt[2 * TM * BP];  // exp(gam) q
    float* sG = reinterpret_cast<float*>(sKt);  // fp32 g rows [TM][KP] until then
    __shared__ __attribute__((aligned(16))) float sA[TM * AP];   // split h0 columns [j][c], then A
    __shared__ __attribute__((aligned(16))) float sP[TM * AP];   // v columns [j][t], then P
    __shared__ __attribute__((aligned(16))) float sU[TM * UP];   // right-hand side, then U
    __shared__ unsigned long long sAnc[TM];
    __shared__ float sBeta[TM];

    // blocks: (batch, value head, group of ncbw column blocks of CB v columns)
    const int ngrp = DV / CB / ncbw;
    const int grp = blockIdx.x % ngrp;
    const int bh = blockIdx.x / ngrp;
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int hg = h / (HV / HG);  // gate head
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int T16 = (T + 15) & ~15;
    const int NB = T16 / 16;
    const int col0 = grp * ncbw * CB;  // the first block's columns

    // ---- 0. global reads, all requested before any is used --------------------------------
    // Issued in the order they are needed: parents and beta, then g (the decay prefixes need
    // only these), then k, q, the v tile and the h0 columns, which stay in flight through
    // the masks and prefixes (their barriers wait for LDS traffic only).  Every thread issues
    // the same straight-line loads (rows past the tree read row T - 1 and are zeroed), so
    // each use waits for exactly the loads issued before its own.
    const int tp = min(lane, T - 1);
    const int par = parent[(size_t)b * T + tp];
    const float bta = beta[((size_t)b * T + tp) * HV + h];
    // g/k/q: thread t covers 4 channels of rows t / (DK/4) + (256 / (DK/4)) * m
    constexpr int QPR = DK / 4;            // 4-channel groups per row
    constexpr int RPI = 256 / QPR;         // rows per pass
    constexpr int NPASS = TM / RPI;
    const int c4 = 4 * (tid % QPR);
    f32x4 gv[NPASS];
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {
        const int t = min(tid / QPR + RPI * m, T - 1);
        gv[m] = load_g4(g, (((size_t)b * T + t) * HG + hg) * DK + c4);
        if constexpr (GS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gv[m][e] = neg_softplus(gv[m][e]);
        }
    }
    uint32_t kraw[NPASS][ELT], qraw[NPASS][ELT];
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {
        const int t = min(tid / QPR + RPI * m, T - 1);
        const size_t kq = (((size_t)b * T + t) * HK + kh) * DK + c4;
        if constexpr (ELT == 2) {
            const uint2 kk = *reinterpret_cast<const uint2*>(k + kq);
            const uint2 qq = *reinterpret_cast<const uint2*>(q + kq);
            kraw[m][0] = kk.x; kraw[m][1] = kk.y;
            qraw[m][0] = qq.x; qraw[m][1] = qq.y;
        } else {
            const uint4 kk = *reinterpret_cast<const uint4*>(k + kq);
            const uint4 qq = *reinterpret_cast<const uint4*>(q + kq);
            kraw[m][0] = kk.x; kraw[m][1] = kk.y; kraw[m][2] = kk.z; kraw[m][3] = kk.w;
            qraw[m][0] = qq.x; qraw[m][1] = qq.y; qraw[m][2] = qq.z; qraw[m][3] = qq.w;
        }
    }
    // v rows: thread covers node t = tid / 8 + 32 m, 4 columns
    uint32_t vraw[2][ELT];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int t = min(tid / 8 + 32 * m, T - 1);
        const size_t vo = (((size_t)b * T + t) * HV + h) * DV + col0 + 4 * (tid % 8);
        if constexpr (ELT == 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(v + vo);
            vraw[m][0] = x.x; vraw[m][1] = x.y;
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(v + vo);
            vraw[m][0] = x.x; vraw[m][1] = x.y; vraw[m][2] = x.z; vraw[m][3] = x.w;
        }
    }
    // h0 columns col0 .. col0+31: thread covers row c = tid / 8 + 32 m, 4 columns.  Buffer
    // loads over this head's state, of range 0 without h0 (they then read zeros), so the
    // loads are issued unconditionally.
    constexpr int HPASS = DK / 32;
    const rsrc_t rs_h0 = make_rsrc(h0 != nullptr ? h0 + (size_t)bh * DK * DV : nullptr,
                                   h0 != nullptr ? (uint32_t)(DK * DV * 4) : 0u);
    f32x4 hv[HPASS];
#pragma unroll
    for (int m = 0; m < HPASS; ++m)
        hv[m] = buf_load_f32x4(rs_h0, ((tid / 8 + 32 * m) * DV + col0 + 4 * (tid % 8)) * 4, 0);
    // ---- 1. ancestor masks, then the decay prefixes ---------------------------------------
    // Wave 0, one node per lane, doubles parent pointers in registers (lane shuffles, no
    // workgroup barrier): after round r, J is the node 2^r steps up (-1 past the root) and
    // anc holds the 2^r nearest strict ancestors.  A tree of depth below 2^r needs r rounds;
    // the ballot makes the exit wave-uniform.
    if (wave == 0) {
        int J = lane < T ? par : -1;
        if (J < -1 || J >= lane) J = -1;  // not an earlier node: a child of the initial state
        unsigned long long anc = J >= 0 ? 1ull << J : 0ull;
        for (int round = 0; round < 6 && __ballot(J >= 0) != 0ull; ++round) {
            const int src = J >= 0 ? J : lane;
            const int jj = __shfl(J, src);
            const uint32_t alo = __shfl((uint32_t)anc, src);
            const uint32_t ahi = __shfl((uint32_t)(anc >> 32), src);
            if (J >= 0) {
                anc |= ((unsigned long long)ahi << 32) | alo;
                J = jj;
            }
        }
        sAnc[lane] = anc;
        sBeta[lane] = lane < T ? bta : 0.f;
    }
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {  // g rows, zero past the tree
        const int t = tid / QPR + RPI * m;
        if (t >= T) gv[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(sG + t * KP + c4) = gv[m];
    }
    lds_barrier();
    // gam = M g with M[t][s] = 1 for s = t or an ancestor of t (0 past the tree): fp32 matrix
    // cores, rows of tile I reducing over s < 16 (I + 1) only; wave w takes the 16-channel
    // tiles w (and w + 4), all four row tiles of each as straight-line code so every read is
    // issued before the products (tiles past the tree have all-zero masks).  Every prefix is
    // a plain fp32 sum of its path's g values.
    float* sGam = reinterpret_cast<float*>(sKh);  // [TM][KP], free until the decayed rows
    if (wave < DK / 16) {
        constexpr int NCT = DK / 16 > 4 ? 2 : 1;  // channel tiles per wave
        unsigned long long bits[4];  // this lane's row of M, from the lane group's first column
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const int t = 16 * I + li;
            bits[I] = (t < T ? (sAnc[t] | (1ull << t)) : 0ull) >> (gq * 4 * (I + 1));
        }
        f32x4 acc[NCT][4];
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const float* yc = sG + 16 * (wave + 4 * u) + li;
            acc[u][0] = prefix_tile<4>(bits[0], yc + gq * 4 * KP, KP);
            acc[u][1] = prefix_tile<8>(bits[1], yc + gq * 8 * KP, KP);
            acc[u][2] = prefix_tile<12>(bits[2], yc + gq * 12 * KP, KP);
            acc[u][3] = prefix_tile<16>(bits[3], yc + gq * 16 * KP, KP);
        }
#pragma unroll
        for (int u = 0; u < NCT; ++u)
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sGam[(16 * I + 4 * gq + i) * KP + 16 * (wave + 4 * u) + li] = acc[u][I][i];
    }
    lds_barrier();
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {
        const int t = tid / QPR + RPI * m;
        gv[m] = *reinterpret_cast<const f32x4*>(sGam + t * KP + c4);
    }
    lds_barrier();  // every prefix is read before the decayed rows overwrite sKh
    auto raw4 = [&](const uint32_t (&r)[ELT]) {
        f32x4 x;
        if constexpr (ELT == 2) {
            x[0] = __uint_as_float(r[0] << 16); x[1] = __uint_as_float(r[0] & 0xFFFF0000u);
            x[2] = __uint_as_float(r[1] << 16); x[3] = __uint_as_float(r[1] & 0xFFFF0000u);
        } else {
            x[0] = __uint_as_float(r[0]); x[1] = __uint_as_float(r[1]);
            x[2] = __uint_as_float(r[2]); x[3] = __uint_as_float(r[3]);
        }
        return x;
    };
    // decayed rows, from the prefixes and the k and q rows still in registers, stored as
    // bf16 high/low pairs over the g rows and the prefixes (both read before the last
    // barrier)
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {
        const int t = tid / QPR + RPI * m;
        const int i = t * BP + c4;
        // rows past the tree: zero keys and queries (their prefixes are 0), so every
        // decayed value is +0
        uint32_t kr[ELT], qr[ELT];
#pragma unroll
        for (int e = 0; e < ELT; ++e) {
            kr[e] = t < T ? kraw[m][e] : 0u;
            qr[e] = t < T ? qraw[m][e] : 0u;
        }
        f32x4 kv = raw4(kr);
        const f32x4 qv = raw4(qr);
        if constexpr (KN) {  // the row's dk entries sit in QPR consecutive lanes
            float s2 = kv[0] * kv[0] + kv[1] * kv[1] + kv[2] * kv[2] + kv[3] * kv[3];
#pragma unroll
            for (int off = 1; off < QPR; off <<= 1) s2 += __shfl_xor(s2, off);
            kv *= inv_key_norm(s2);
        }
        f32x4 kt, kb, qt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ep = __expf(gv[m][e]);
            kt[e] = ep * kv[e];
            kb[e] = __expf(-gv[m][e]) * kv[e];
            qt[e] = ep * qv[e];
        }
        bf16x4 hi, lo;
        split4(kt, hi, lo);
        *reinterpret_cast<bf16x4*>(sKt + i) = hi;
        *reinterpret_cast<bf16x4*>(sKt + LO + i) = lo;
        split4(kb, hi, lo);
        *reinterpret_cast<bf16x4*>(sKh + i) = hi;
        *reinterpret_cast<bf16x4*>(sKh + LO + i) = lo;
        split4(qt, hi, lo);
        *reinterpret_cast<bf16x4*>(sQt + i) = hi;
        *reinterpret_cast<bf16x4*>(sQt + LO + i) = lo;
    }
    // Per column block: stage its h0 columns (transposed, bf16 high/low pairs: high [CB][BP]
    // then low [CB][BP]) and its v tile (transposed, fp32 [CB][TM + 4]) from registers
    auto stage = [&](const f32x4 (&hvv)[HPASS], const uint32_t (&vr)[2][ELT], __bf16* sH, float* sVt) {
#pragma unroll
        for (int m = 0; m < HPASS; ++m) {  // sH[j * BP + c]
            const int c = tid / 8 + 32 * m;
            bf16x4 hi, lo;
            split4(hvv[m], hi, lo);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sH[(4 * (tid % 8) + e) * BP + c] = hi[e];
                sH[CB * BP + (4 * (tid % 8) + e) * BP + c] = lo[e];
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {  // sVt[j * (TM + 4) + t]
            const int t = tid / 8 + 32 * m;
            const f32x4 x = raw4(vr[m]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sVt[(4 * (tid % 8) + e) * (TM + 4) + t] = t < T ? x[e] : 0.f;
        }
    };
    // the global reads of the column block starting at column colb (h0 columns, v tile)
    auto load_block = [&](int colb, f32x4 (&hvv)[HPASS], uint32_t (&vr)[2][ELT]) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = min(tid / 8 + 32 * m, T - 1);
            const size_t vo = (((size_t)b * T + t) * HV + h) * DV + colb + 4 * (tid % 8);
            if constexpr (ELT == 2) {
                const uint2 x = *reinterpret_cast<const uint2*>(v + vo);
                vr[m][0] = x.x; vr[m][1] = x.y;
            } else {
                const uint4 x = *reinterpret_cast<const uint4*>(v + vo);
                vr[m][0] = x.x; vr[m][1] = x.y; vr[m][2] = x.z; vr[m][3] = x.w;
            }
        }
#pragma unroll
        for (int m = 0; m < HPASS; ++m)
            hvv[m] = buf_load_f32x4(rs_h0, ((tid / 8 + 32 * m) * DV + colb + 4 * (tid % 8)) * 4, 0);
    };

    // ---- 2. Kt h0, Qt h0 and the right-hand side beta (v - Kt h0) -------------------------
    // tile (I, N): rows 16I.., columns 16N.. of the block; wave w owns tiles w and w + 4 and
    // keeps its Qt h0 tiles for the output
    auto rhs = [&](const __bf16* sH, const float* sVt, f32x4 (&qh)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = wave + 4 * u;
            f32x4 kacc = {0.f, 0.f, 0.f, 0.f}, qacc = {0.f, 0.f, 0.f, 0.f};
            if (tile < 2 * NB) {
                const int I = tile >> 1, N = tile & 1;
                const int cq = 8 * gq;
                const __bf16* hb = sH + (16 * N + li) * BP + cq;
                kacc = tile_dot_split<DK>(sKt + (16 * I + li) * BP + cq, LO, hb, CB * BP);
                qacc = tile_dot_split<DK>(sQt + (16 * I + li) * BP + cq, LO, hb, CB * BP);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * gq + i;
                    sU[r * UP + 16 * N + li] = sBeta[r] * (sVt[(16 * N + li) * (TM + 4) + r] - kacc[i]);
                }
            }
            qh[u] = qacc;
        }
    };

    // ---- 4. (I + A) U = rhs by 16-row blocks ----------------------------------------------
    // A_rs is nonzero only for s an ancestor of r, so s < r: I + A is unit lower triangular
    // and so is each diagonal block D_I.  Lane (block gq, column li) runs forward
    // substitution down column li of inv(D_gq) in registers; then block by block
    //   U_I = inv(D_I) R_I,  R_J <- R_J - A_JI U_I  for J > I   (R starts as the rhs)
    // with both products on the matrix cores, so U_I = inv(D_I) (rhs_I - sum_{J<I} A_IJ U_J).
    constexpr int DIP = 20;            // inverse row pitch: 16-byte reads of 16 rows, no conflict
    constexpr int DIB = 16 * DIP + 16; // inverse block stride
    static_assert(4 * DIB * 4 <= 2 * TM * BP * 2, "block inverses must fit the free key rows");
    auto invert_diag = [&](float* sDi) {
        if (gq < NB) {
            const float* ab = sA + 16 * gq * AP + 16 * gq;  // diagonal block gq
            float xc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == li ? 1.f : 0.f;
#pragma unroll
                for (int q4 = 0; q4 < (r + 3) / 4; ++q4) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(ab + r * AP + 4 * q4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q4 + e < r) acc -= a4[e] * xc[4 * q4 + e];
                }
                xc[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sDi[gq * DIB + r * DIP + li] = xc[r];
        }
    };
    // Right-looking block substitution with every operand in registers (waves 0 and 1, one
    // 16-column tile of U each): each block's right-hand side R_I (rows 4 gq + i, column li)
    // and U_I stay in the accumulator layout, which is also the B-operand layout of a
    // 16x16x4 product whose step i pairs reduction slot gq with row 4 gq + i; so U_I feeds
    // the updates R_J -= A_JI U_I (J > I) directly.  All reads are issued first (blocks past
    // the tree are read but never used).
    auto substitute = [&](const float* sDi) {
        const int N = wave;
        f32x4 R[4], di[4], aJI[6];  // aJI: (J, I) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int i = 0; i < 4; ++i) R[I][i] = sU[(16 * I + 4 * gq + i) * UP + 16 * N + li];
            di[I] = *reinterpret_cast<const f32x4*>(sDi + I * DIB + li * DIP + 4 * gq);
        }
#pragma unroll
        for (int J = 1, n = 0; J < 4; ++J)
#pragma unroll
            for (int I = 0; I < J; ++I, ++n)
                aJI[n] = *reinterpret_cast<const f32x4*>(sA + (16 * J + li) * AP + 16 * I + 4 * gq);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I < NB) {
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) u = mfma4(di[I][i], R[I][i], u);
#pragma unroll
                for (int i = 0; i < 4; ++i) sU[(16 * I + 4 * gq + i) * UP + 16 * N + li] = u[i];
#pragma unroll
                for (int J = I + 1; J < 4; ++J) {
                    if (J < NB) {
                        const f32x4 a = aJI[J * (J - 1) / 2 + I];
#pragma unroll
                        for (int i = 0; i < 4; ++i) R[J] = mfma4(-a[i], u[i], R[J]);
                    }
                }
            }
        }
    };

    // ---- 5. O = Qt h0 + P U ----------------------------------------------------------------
    auto outputs = [&](const f32x4 (&qh)[2], int colb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = wave + 4 * u;
            if (tile < 2 * NB) {
                const int I = tile >> 1, N = tile & 1;
                // P's row tile I is zero right of its diagonal tile: reduce over s < 16 (I + 1),
                // lane group gq taking 4 (I + 1) of them
                f32x4 acc = qh[u];
                const float* rp = sP + (16 * I + li) * AP + gq * 4 * (I + 1);
                const float* ub = sU + gq * 4 * (I + 1) * UP + 16 * N + li;
                if (I == 0) acc = tile_rows_cols<4>(rp, ub, UP, acc);
                else if (I == 1) acc = tile_rows_cols<8>(rp, ub, UP, acc);
                else if (I == 2) acc = tile_rows_cols<12>(rp, ub, UP, acc);
                else acc = tile_rows_cols<16>(rp, ub, UP, acc);
                const int col = colb + 16 * N + li;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * gq + i;
                    if (r < T) store_o1(o, (((size_t)b * T + r) * HV + h) * DV + col, acc[i], obf);
                }
            }
        }
    };

    // Several column blocks per workgroup only where the diagonal inverses and one staged
    // block fit the key rows freed once A and P are formed (dk = 128); the host asks for
    // one otherwise.
    constexpr int DIP0 = 20, DIB0 = 16 * DIP0 + 16;
    constexpr bool kMulti = 4 * DIB0 * 4 + 2 * CB * BP * 2 + CB * (TM + 4) * 4 <= 2 * TM * BP * 2;
    const int nblk_w = kMulti ? ncbw : 1;

    // The first column block: its h0 columns in sA's memory and its v tile in sP's, both
    // dead once A and P are formed; the next block's reads are issued as soon as the
    // registers are free, so they are in flight through this block.
    stage(hv, vraw, reinterpret_cast<__bf16*>(sA), sP);
    if (nblk_w > 1) load_block(col0 + CB, hv, vraw);
    lds_barrier();  // decayed rows, h0 columns and v tile (read across threads below)
    f32x4 qh[2];
    rhs(reinterpret_cast<const __bf16*>(sA), sP, qh);
    lds_barrier();

    // ---- 3. A and P tiles, masked by ancestry (upper tiles are zero) -----------------------
    // Only the NB(NB+1)/2 lower tiles of each hold products; they are dealt evenly to the
    // waves.  The upper tiles are never read (the solve and the output product reduce over
    // the lower ones only).
    const int nlow = NB * (NB + 1) / 2;  // <= 10 (NB <= 4)
    for (int job = wave; job < 2 * nlow; job += 4) {
        const int x = job >= nlow;  // 0: A, 1: P
        const int t = job - x * nlow;
        const int I = (t >= 1) + (t >= 3) + (t >= 6);  // lower tile t = I (I + 1) / 2 + J
        const int J = t - I * (I + 1) / 2;
        float* dst = x == 0 ? sA : sP;
        const int cq = 8 * gq;
        const int s = 16 * J + li;
        // the rows' ancestor masks and betas are read before the products, so their LDS
        // round trips overlap the matrix-core work
        unsigned long long am[4];
        float bt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i;
            am[i] = sAnc[r];
            bt[i] = sBeta[r];
        }
        const f32x4 acc = tile_dot_split<DK>((x == 0 ? sKt : sQt) + (16 * I + li) * BP + cq, LO,
                                             sKh + (16 * J + li) * BP + cq, LO);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i;
            const bool anc = (am[i] >> s) & 1ull;
            float val;
            if (x == 0) val = anc ? bt[i] * acc[i] : 0.f;
            else val = (anc || s == r) ? acc[i] : 0.f;
            if (r >= T || s >= T) val = 0.f;
            dst[r * AP + s] = val;
        }
    }
    lds_barrier();

    // The diagonal inverses.  With one column block, waves 0 and 1 each invert every
    // diagonal block into a private copy (sKt or sKh, both free now), so no barrier separates
    // the inversion from its use.  With several, the decayed keys and queries stay live for
    // the later blocks: wave 0 writes the one copy at the start of sKh, followed by the
    // later blocks' staged h0 columns and v tiles.
    float* sInv = reinterpret_cast<float*>(sKh);
    __bf16* sHn = reinterpret_cast<__bf16*>(sInv + 4 * DIB);
    float* sVn = reinterpret_cast<float*>(sHn + 2 * CB * BP);
    static_assert(DIB == DIB0, "one inverse layout");
    if (nblk_w == 1) {
        if (wave < 2) {
            float* sDi = reinterpret_cast<float*>(wave == 0 ? sKt : sKh);
            invert_diag(sDi);
            substitute(sDi);
        }
    } else {
        if (wave == 0) invert_diag(sInv);
        lds_barrier();
        if (wave < 2) substitute(sInv);
    }
    lds_barrier();
    outputs(qh, col0);

    // Later column blocks (several per workgroup when there are enough heads to fill the
    // chip): the decayed rows, A, P and the inverses are reused.
    for (int j = 1; j < nblk_w; ++j) {
        stage(hv, vraw, sHn, sVn);
        if (j + 1 < nblk_w) load_block(col0 + (j + 1) * CB, hv, vraw);
        lds_barrier();  // staged block; the previous block's outputs have read sU
        rhs(sHn, sVn, qh);
        lds_barrier();
        if (wave < 2) substitute(sInv);
        lds_barrier();
        outputs(qh, col0 + j * CB);
    }
}

// Column blocks per workgroup: with enough (batch, value head, column block) triples for
// several rounds of workgroups, a workgroup takes 2 or 4 blocks of one head and forms the
// decayed rows, A, P and the diagonal inverses once for all of them, as long as the
// workgroups still fill the 256 CUs (dk = 128 only; see the kernel).
inline int tree_blocks_per_group(long long B, int HV, int ncb, int dk) {
    if (dk != 128) return 1;
    for (int w : {4, 2})
        if (ncb % w == 0 && B * HV * (ncb / w) >= 256) return w;
    return 1;
}

template <typename TIn, typename TG, int DK, bool KN, bool GS>
hipError_t launch_tree_t(const LaunchArgs& a, const int32_t* parent) {
    const int ncb = a.dv / CB;
    const int ncbw = tree_blocks_per_group(a.B, a.HV, ncb, DK);
    const long long nblk = (long long)a.B * a.HV * (ncb / ncbw);
    hipLaunchKernelGGL((tree_verify_kernel<TIn, TG, DK, KN, GS>), dim3((unsigned)nblk), dim3(256), 0,
                       (hipStream_t)a.stream, parent, (const TIn*)a.q, (const TIn*)a.k,
                       (const TIn*)a.v, (const TG*)a.g, a.beta, a.h0, a.o, a.T, a.HK, a.HV, a.HG, a.dv, ncbw,
                       (int)a.o_bf16);
    return hipGetLastError();
}

template <typename TIn, typename TG, bool KN, bool GS>
hipError_t dispatch_tree(const LaunchArgs& a, const int32_t* parent) {
    if (a.dk == 32) return launch_tree_t<TIn, TG, 32, KN, GS>(a, parent);
    if (a.dk == 64) return launch_tree_t<TIn, TG, 64, KN, GS>(a, parent);
    if (a.dk == 128) return launch_tree_t<TIn, TG, 128, KN, GS>(a, parent);
    return hipErrorInvalidValue;
}

template <bool KN, bool GS>
hipError_t dispatch_tree_types(const LaunchArgs& a, const int32_t* parent) {
    if (a.qkv_f32) return dispatch_tree<float, float, KN, GS>(a, parent);
    return a.g_bf16 ? dispatch_tree<bf16_t, bf16_t, KN, GS>(a, parent) : dispatch_tree<bf16_t, float, KN, GS>(a, parent);
}

}  // namespace

hipError_t launch_tree_verify(const LaunchArgs& a, const int32_t* parent) {
    if (a.T < 1 || a.T > TM || a.dv % CB != 0) return hipErrorInvalidValue;
    if (a.k_l2norm)
        return a.g_softplus ? dispatch_tree_types<true, true>(a, parent) : dispatch_tree_types<true, false>(a, parent);
    return a.g_softplus ? dispatch_tree_types<false, true>(a, parent) : dispatch_tree_types<false, false>(a, parent);
}

}  // namespace gdr
