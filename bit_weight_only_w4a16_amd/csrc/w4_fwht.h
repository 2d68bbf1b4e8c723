// w4_fwht.h -- butterfly stages of the blockwise Walsh-Hadamard transform,
// shared by the transform kernel and the kernels that fuse it (internal).
//
// [P2] "fastgemma -- Gemma 4 E2B, CPU-only, AMX INT8 / AVX-512 VNNI", section
// "What is in the file": the activations get a fast Walsh-Hadamard transform
// at run time.  Sylvester order; the caller applies the orthonormal scale
// block^-1/2 once at the end, so every user rounds identically.
#pragma once

#include "w4_common.h"

namespace w4 {

// One block held E values per lane: lane l holds elements l*E .. l*E + E - 1
// of a block of lanes * E (lanes <= 64).  Spans below E stay inside a lane;
// span h >= E pairs lane l with lane l ^ (h / E).  fp32, in place.
template <int E>
__device__ __forceinline__ void fwht_block(float (&v)[E], int lane, int lanes) {
#pragma unroll
    for (int h = 1; h < E; h *= 2) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & h) == 0) {
                const float a = v[e], c = v[e + h];
                v[e] = a + c;
                v[e + h] = a - c;
            }
        }
    }
    for (int d = 1; d < lanes; d *= 2) {
        const bool upper = (lane & d) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float o = __shfl_xor(v[e], d, 64);
            v[e] = upper ? (o - v[e]) : (v[e] + o);
        }
    }
}

}  // namespace w4
