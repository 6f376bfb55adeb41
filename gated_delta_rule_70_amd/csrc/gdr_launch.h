// Internal interface between the host entry points (gdr_api.cpp) and the kernel launchers
// (one .hip file per kernel family).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

struct LaunchArgs {
    int B, T, HK, HV, dk, dv, chunk;
    bool qkv_f32;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* h0;
    float* o;
    float* ht;
    void* workspace;
    void* stream;
};

// Per-(batch, head, chunk) record that the chunk-parallel kernel writes and the
// sequential carry kernel reads: fp16 MFMA operand fragments (1 KiB each: 64 lanes x 8
// halves, lane-major) followed by one 1 KiB block whose first dk floats hold the chunk's
// total decay exp(gam_last).  Records are a whole number of KiB so the carry kernel can
// stream one into LDS with 1 KiB wave-wide copies.
//   Qt  [nb][kc]    decayed queries exp(gam) * q           (rows r, reduction over dk)
//   -W  [nb][kc]    negated WY pseudo-keys                  (rows r, reduction over dk)
//   Kb  [dkt][nqs]  decay-to-end keys, transposed           (rows c, reduction over tokens)
//   Tb  [nb][nqs]   Tinv diag(beta)                         (rows r, reduction over tokens)
//   P   [nb][nqs]   causal q.k terms                        (rows r, reduction over tokens)
// Tb and P are lower triangular: the slots of their all-zero fragments (token steps above
// a row tile's diagonal) are left unwritten, and the carry reads them as zeros from
// beyond the buffer range, so every row tile issues the same operand loads.
struct ChunkRecord {
    int nb;        // 16-row blocks per chunk (C / 16)
    int nqs;       // 32-wide token reduction steps (ceil(C / 32))
    int kc;        // 32-wide key-channel reduction steps (dk / 32)
    int dkt;       // 16-row key-channel tiles (dk / 16)
    int off_qt;    // fragment offsets (in fragments) of each operand
    int off_w;
    int off_kb;
    int off_tb;
    int off_p;
    int nfrag;     // operand fragments; the decay block follows them
    int bytes;     // record stride: (nfrag + 1) KiB

    __host__ __device__ static constexpr ChunkRecord make(int C, int dk) {
        ChunkRecord r{};
        r.nb = C / 16;
        r.nqs = (C + 31) / 32;
        r.kc = dk / 32;
        r.dkt = dk / 16;
        r.off_qt = 0;
        r.off_w = r.off_qt + r.nb * r.kc;
        r.off_kb = r.off_w + r.nb * r.kc;
        r.off_tb = r.off_kb + r.dkt * r.nqs;
        r.off_p = r.off_tb + r.nb * r.nqs;
        r.nfrag = r.off_p + r.nb * r.nqs;
        r.bytes = (r.nfrag + 1) * 1024;
        return r;
    }
};

// token recurrence over a.T tokens in one launch (the decode step is a.T == 1)
hipError_t launch_tokens(const LaunchArgs& a);
hipError_t launch_chunk_prep(const LaunchArgs& a);
hipError_t launch_chunk_carry(const LaunchArgs& a);
// tree-verify solve over trees of a.T <= 64 nodes; parent [B][T] int32 on the device
hipError_t launch_tree_verify(const LaunchArgs& a, const int32_t* parent);

}  // namespace gdr
