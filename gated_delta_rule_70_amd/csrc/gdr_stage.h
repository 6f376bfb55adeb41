// Internal helpers shared by the carry kernels: the LDS layout of a staged chunk record,
// the list of record fragments a carry copies, and the bookkeeping of the power-of-two
// scaled domains that keep the carry's fp16 operands in range.
#pragma once

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

// Scale bookkeeping of the wave's scaled domain: values are kept with their largest
// magnitude at most 2^kTop (U = Tb V - W X' then stays below 2^kTop (|Tb|_1 + |W|_1), far
// inside fp16) and rescaled to [2^(kTop-1), 2^kTop) once it exceeds that or falls below
// 2^(kTop-kSlack).  kNoExp: the state and v are zero so far.
constexpr int kTop = 6;
constexpr int kSlack = 10;
constexpr int kNoExp = -1000;

// Largest |x| over raw v bits (bf16 pairs or fp32), as a packed/unpacked running maximum.
typedef unsigned short u16x2w __attribute__((ext_vector_type(2)));
template <typename TIn>
struct VMax {
    u16x2w m16 = {0, 0};
    float m32 = 0.f;
    __device__ __forceinline__ void add(uint32_t x) {
        if constexpr (sizeof(TIn) == 2)
            m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(u16x2w, x & 0x7FFF7FFFu));
        else
            m32 = fmaxf(m32, fabsf(__uint_as_float(x)));
    }
    __device__ __forceinline__ float get() const {
        if constexpr (sizeof(TIn) == 2) return __uint_as_float((uint32_t)(m16[0] > m16[1] ? m16[0] : m16[1]) << 16);
        return m32;
    }
};

// LDS layout of one staged record (slots of 1 KiB, lane-major fragments) and the list of
// record fragments copied into it.  Tb and P fragments above a row tile's diagonal are
// zero, are not written by chunk_prep and are never copied or read.  The summary pass
// needs neither Qt nor P.
template <int C, int D, bool SUM>
struct Stage {
    static constexpr ChunkRecord R = ChunkRecord::make(C, D);
    static constexpr int NB = C / 16, NQS = (C + 31) / 32, KC = D / 32, DKT = D / 16;
    static constexpr int s_w = 0;
    static constexpr int s_kb = s_w + NB * KC;
    static constexpr int s_tb = s_kb + DKT * NQS;
    static constexpr int s_qt = s_tb + NB * NQS;
    static constexpr int s_p = s_qt + (SUM ? 0 : NB * KC);
    static constexpr int s_e = s_p + (SUM ? 0 : NB * NQS);
    static constexpr int nslot = s_e + 1;
};

struct CopyList {
    int n;
    short id[96];
    short slot[96];
};

template <int C, int D, bool SUM>
constexpr CopyList make_copy_list() {
    using S = Stage<C, D, SUM>;
    constexpr ChunkRecord R = S::R;
    CopyList l{};
    auto add = [&](int id, int slot) {
        l.id[l.n] = (short)id;
        l.slot[l.n] = (short)slot;
        ++l.n;
    };
    for (int i = 0; i < S::NB * S::KC; ++i) add(R.off_w + i, S::s_w + i);
    for (int i = 0; i < S::DKT * S::NQS; ++i) add(R.off_kb + i, S::s_kb + i);
    for (int r = 0; r < S::NB; ++r)
        for (int qs = 0; 2 * qs <= r && qs < S::NQS; ++qs) add(R.off_tb + r * S::NQS + qs, S::s_tb + r * S::NQS + qs);
    if (!SUM) {
        for (int i = 0; i < S::NB * S::KC; ++i) add(R.off_qt + i, S::s_qt + i);
        for (int r = 0; r < S::NB; ++r)
            for (int qs = 0; 2 * qs <= r && qs < S::NQS; ++qs) add(R.off_p + r * S::NQS + qs, S::s_p + r * S::NQS + qs);
    }
    add(R.nfrag, S::s_e);  // exp(gam_last) block
    return l;
}

}  // namespace gdr
