// w4_attn.hip -- split-K decode attention: one key/value head, eight query heads.
//
// [P1] "Gemma 4 E2B on a 4 GB GPU with plain PyTorch, faster than llama.cpp",
// paragraph on w4attn.py: the model has one key/value head shared by eight
// query heads, so each cached key and value is read once for all eight heads,
// the cache is split into slices, and the slices are combined with an online
// softmax; paragraph on the cache: full layers hold one slot per position
// (head width 512), sliding layers a 512-slot ring that records each slot's
// position, and masks are built from positions.
//
// MI355X shape of it.  Per 32-slot tile, both products run on the matrix
// cores (v_mfma_f32_16x16x32_bf16, heads padded to 16):
//   S^T = K Q^T   A = 16 key rows x 32 dims, B = Q^T (dims x heads),
//   O^T += V^T P^T  A = 16 dims x 32 slots of V^T, B = P^T (slots x heads).
// Key rows are read in their natural layout; the score tile leaves every lane
// with one head and 8 slots, which is exactly the B operand of the second
// product, so P needs no transpose.  V is stored in 32-slot blocks, each D
// rows of 32 slots (the blocked layout w4_attn_pack_v writes), so the A
// operand of the second product is one 16-byte load per lane.
// The four waves of a workgroup split the head width D into quarters: each
// computes partial scores over its quarter, the partials are summed through
// LDS in a fixed order (identical in every wave), the softmax bookkeeping is
// repeated in every wave, and each wave accumulates O for its quarter of D
// only.  A workgroup walks a contiguous range of tiles and writes one partial
// (running max, running sum, unnormalised O); a second kernel merges the
// partials of all workgroups.
#include "w4_dispatch.h"

namespace w4 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int kAttnHeads = 8;
constexpr int kAttnTile = 32;
// split workgroups, at most: one per CU (measured at D = 512: 131072 slots
// 48.0 -> 45.5 us, 32768 slots 21.3 -> 17.8 us against two per CU; three per
// CU were slower still): fewer partials for the merge to read
constexpr int kAttnMaxWG = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const uint16_t* q;    // [8][D]
    const uint16_t* K;    // [T][ldk]
    const uint16_t* Vt;   // blocked: tile b, dim d, slot c at ((b * D + d) * 32 + c)
    const int32_t* pos;   // nullptr or [T]
    float* part;          // per workgroup: m[16], l[16], O[8][D]
    int ldk, T, cur, window, tiles, nwg;
    float scale2;         // scale * log2(e): scores in base 2
};

__device__ __forceinline__ int part_stride(int D) { return 32 + kAttnHeads * D; }

// Slot c is attended iff c < T and, with positions, the slot's position p is
// in (cur - window, cur] (window 0: no lower bound).
template <bool POS>
__device__ __forceinline__ bool slot_valid(const AttnArgs& a, int c, int p) {
    if (c >= a.T) return false;
    if (!POS) return true;
    return p >= 0 && p <= a.cur && (a.window <= 0 || p > a.cur - a.window);
}

}  // namespace

// POS: the cache records a position per slot (ring caches).  Every load of a
// tile is unconditional (indices clamped into the cache; slots past T are
// rejected by slot_valid), so the compiler can count the loads in flight
// exactly and keeps the next tile's loads outstanding across the loop.
template <int D, bool POS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_split_kernel(AttnArgs a) {
    constexpr int DQ = D / 4;   // dims per wave
    constexpr int KS = DQ / 32; // score k-steps per wave
    constexpr int DT = DQ / 16; // output tiles (16 dims) per wave
    __shared__ float sx[2][4][8][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;  // head (columns of both products)
    const int g = lane >> 4;  // k-group of the operands, row group of the results
    const int d0 = wave * DQ;
    const int tb = (int)((long long)a.tiles * blockIdx.x / a.nwg);
    const int te = (int)((long long)a.tiles * (blockIdx.x + 1) / a.nwg);

    // B operand of S^T = K Q^T: head i, dims d0 + 32 s + 8 g .. + 7 (zero for padded heads)
    u32x4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (i < kAttnHeads)
            qf[s] = gload(reinterpret_cast<const u32x4*>(a.q + (size_t)i * D + d0 + 32 * s + 8 * g));
        else
            qf[s] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;

    // One register set per tile part, reloaded for the next tile as soon as
    // the part has been consumed: keys (and positions) right after the score
    // products, values right after the PV product.  Each load then has about
    // half a tile of work to hide behind, with half the registers of a
    // two-set ping-pong (whose register reuse made the compiler drain every
    // load at each tile).  The last tile reloads itself, so every load is
    // unconditional and every wait counts exactly.
    // Score tile a row r is slot p0 + 8 (r / 4) + r % 4, tile b that + 4, so
    // result row 4 g + j holds slot p0 + 8 g + j (tile a, j < 4) or + 4 (tile
    // b); V^T rows are dims d0 + 16 t + i, slots 8 g .. 8 g + 7.
    u32x4 ka[KS], kb[KS], vf[DT];
    int pos[8];
    auto load_k = [&](int tau) {
        const int p0 = tau * kAttnTile;
        const int ra = p0 + 8 * (i >> 2) + (i & 3);
        const int rb = ra + 4;
        const uint16_t* kra = a.K + (size_t)(ra < a.T ? ra : a.T - 1) * a.ldk + d0 + 8 * g;
        const uint16_t* krb = a.K + (size_t)(rb < a.T ? rb : a.T - 1) * a.ldk + d0 + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            ka[s] = gload(reinterpret_cast<const u32x4*>(kra + 32 * s));
            kb[s] = gload(reinterpret_cast<const u32x4*>(krb + 32 * s));
        }
        if (POS) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = p0 + 8 * g + j;
                pos[j] = gload(a.pos + (c < a.T ? c : a.T - 1));
            }
        }
    };
    auto load_v = [&](int tau) {
        const uint16_t* vb =
            a.Vt + (size_t)tau * D * kAttnTile + (size_t)(d0 + i) * kAttnTile + 8 * g;
#pragma unroll
        for (int t = 0; t < DT; ++t)
            vf[t] = gload(reinterpret_cast<const u32x4*>(vb + (size_t)16 * t * kAttnTile));
    };

    load_k(tb);
    load_v(tb);
    for (int tau = tb; tau < te; ++tau) {
        const int nxt = tau + 1 < te ? tau + 1 : tau;
        const int p0 = tau * kAttnTile;
        bool valid[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) valid[j] = slot_valid<POS>(a, p0 + 8 * g + j, POS ? pos[j] : 0);

        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sa = mma(ka[s], qf[s], sa);
            sb = mma(kb[s], qf[s], sb);
        }
        load_k(nxt);
        // partial scores of the four dim quarters: summed in wave order 0..3
        float* buf = &sx[tau & 1][0][0][0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            buf[(wave * 8 + q) * 64 + lane] = sa[q];
            buf[(wave * 8 + 4 + q) * 64 + lane] = sb[q];
        }
        __syncthreads();
        float t8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float sv = ((buf[(0 * 8 + j) * 64 + lane] + buf[(1 * 8 + j) * 64 + lane]) +
                              buf[(2 * 8 + j) * 64 + lane]) +
                             buf[(3 * 8 + j) * 64 + lane];
            t8[j] = valid[j] ? sv * a.scale2 : -__builtin_inff();
        }
        // online softmax of head i over the tile's 32 slots (4 lanes x 8)
        float mt = t8[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mt = fmaxf(mt, t8[j]);
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const bool none = m_new == -__builtin_inff();
        const float alpha = none ? 1.f : exp2f(m_run - m_new);
        uint32_t pb[8];
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float p = none ? 0.f : exp2f(t8[j] - m_new);
            pb[j] = f32_to_bf16_rne(p);
            ls += bf16_to_f32(pb[j]);  // the sum uses the weights the product uses
        }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        l_run = alpha * l_run + ls;
        m_run = m_new;

        const u32x4 pf = u32x4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16),
                               pb[4] | (pb[5] << 16), pb[6] | (pb[7] << 16)};
        // V of slots that are not attended may hold anything (a never-written
        // ring slot, slots past T): zero them so 0 * NaN never reaches O
        u32x4 vmask;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            vmask[w] = (valid[2 * w] ? 0x0000FFFFu : 0u) | (valid[2 * w + 1] ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            acc[t] = acc[t] * alpha;
            acc[t] = mma(vf[t] & vmask, pf, acc[t]);
        }
        load_v(nxt);
    }

    // partial of this workgroup: m and l of each head (base 2), unnormalised O
    float* part = a.part + (size_t)blockIdx.x * part_stride(D);
    if (wave == 0 && g == 0 && i < kAttnHeads) {
        gstore(part + i, m_run);
        gstore(part + 16 + i, l_run);
    }
    if (i < kAttnHeads) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                gstore(part + 32 + i * D + d0 + 16 * t + 4 * g + r, acc[t][r]);
    }
}

// Workgroup-wide reductions over the merge kernel's threads in a fixed tree
// order (the same on every run).
constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 16;                           // dims per merge workgroup
constexpr int kMergeRows = kMergeThreads / kMergeDims;   // partial strides per dim

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int k = kMergeThreads / 2; k > 0; k >>= 1) {
        if ((int)threadIdx.x < k) {
            const float o = red[threadIdx.x + k];
            red[threadIdx.x] = is_max ? fmaxf(red[threadIdx.x], o) : red[threadIdx.x] + o;
        }
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

// out[h][d] = sum_w O_w[h][d] e_w / sum_w l_w e_w, e_w = 2^(m_w - M), M = max_w m_w
// (e_w = 0 for a partial that attended nothing); NaN when no slot was attended.
// Workgroup (h, 16-dim block), 256 threads.  Every load goes out first: thread
// (r, j) takes O of the partials w = r, r + 16, ... (at most 16 * NV partials;
// NV is sized to the launch's partial count) for dim j into registers, and m_w, l_w of its share of partials, so the
// merge costs one memory round trip.  Then M and the weights e_w (once, into
// LDS), the thread's sum in the order w = r, r + 16, ..., and the 16 sums of a
// dim added in order r = 0..15.  (A 16-dim block gives 256 workgroups at
// D = 512, so the partials are read by as many CUs.)
template <int D, int NV>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float* __restrict__ part,
                                                                  int nwg,
                                                                  void* __restrict__ out,
                                                                  int odt) {
    constexpr int S = kMergeRows;
    constexpr int NM = kAttnMaxWG / kMergeThreads;       // (m, l) pairs per thread, at most
    static_assert(NV * S <= kAttnMaxWG && NM * kMergeThreads == kAttnMaxWG, "merge split");
    __shared__ float ew[kAttnMaxWG];
    __shared__ float red[kMergeThreads];
    __shared__ float psum[kMergeRows][kMergeDims];
    const int h = blockIdx.x;
    const int dl = threadIdx.x % kMergeDims;
    const int pr = threadIdx.x / kMergeDims;
    const int d = blockIdx.y * kMergeDims + dl;
    const int ps = part_stride(D);

    const float* col = part + 32 + (size_t)h * D + d;
    float v[NV], mv[NM], lv[NM];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int w = pr + u * S;
        v[u] = w < nwg ? gload(col + (size_t)w * ps) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NM; ++u) {
        const int w = threadIdx.x + u * kMergeThreads;
        mv[u] = w < nwg ? gload(part + (size_t)w * ps + h) : -__builtin_inff();
        lv[u] = w < nwg ? gload(part + (size_t)w * ps + 16 + h) : 0.f;
    }

    float mloc = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < NM; ++u) mloc = fmaxf(mloc, mv[u]);
    const float M = block_reduce(mloc, red, true);
    float lloc = 0.f;
#pragma unroll
    for (int u = 0; u < NM; ++u) {
        const int w = threadIdx.x + u * kMergeThreads;
        const float e = mv[u] == -__builtin_inff() ? 0.f : exp2f(mv[u] - M);
        if (w < nwg) ew[w] = e;
        lloc += lv[u] * e;
    }
    const float L = block_reduce(lloc, red, false);  // ends with a barrier: ew[] complete

    float o = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int w = pr + u * S;
        if (w < nwg) o += v[u] * ew[w];
    }
    psum[pr][dl] = o;
    __syncthreads();
    if (threadIdx.x < kMergeDims) {
        const int t = threadIdx.x;
        float tot = psum[0][t];
#pragma unroll
        for (int k = 1; k < kMergeRows; ++k) tot += psum[k][t];
        const float res = M == -__builtin_inff() ? __builtin_nanf("") : tot / L;
        store_out(out, (size_t)h * D + d, res, odt);
    }
}

// Blocked V: tile b, dim d, slot c at ((b * D + d) * 32 + c); slots past T are 0.
__global__ __launch_bounds__(256) void attn_pack_v_kernel(const uint16_t* __restrict__ V, int ldv,
                                                         int T, int D,
                                                         uint16_t* __restrict__ Vt) {
    const long long row = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // (b, d)
    const int tiles = (T + kAttnTile - 1) / kAttnTile;
    if (row >= (long long)tiles * D) return;
    const int b = (int)(row / D), d = (int)(row - (long long)b * D);
    uint32_t w[16];
#pragma unroll
    for (int c = 0; c < kAttnTile; c += 2) {
        const int t0 = b * kAttnTile + c;
        const uint32_t lo = t0 < T ? gload(V + (size_t)t0 * ldv + d) : 0u;
        const uint32_t hi = t0 + 1 < T ? gload(V + (size_t)(t0 + 1) * ldv + d) : 0u;
        w[c / 2] = lo | (hi << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(Vt + (size_t)row * kAttnTile);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        gstore(dst + k, u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]});
}

// One decode step's cache write: key row `slot` and value column `slot`.
__global__ __launch_bounds__(256) void attn_store_kv_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int slot,
                                                           uint16_t* __restrict__ K, int ldk,
                                                           uint16_t* __restrict__ Vt, int D) {
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        gstore(K + (size_t)slot * ldk + d, gload(k + d));
        gstore(Vt + ((size_t)(slot / kAttnTile) * D + d) * kAttnTile + slot % kAttnTile,
               gload(v + d));
    }
}

// the merge's per-thread O loads: 16 * NV partials cover nwg
template <int D>
static void launch_merge(const float* part, int nwg, void* out, int odt, hipStream_t s) {
    const dim3 g(kAttnHeads, D / kMergeDims), b(kMergeThreads);
    if (nwg <= kMergeRows)
        attn_merge_kernel<D, 1><<<g, b, 0, s>>>(part, nwg, out, odt);
    else if (nwg <= 8 * kMergeRows)
        attn_merge_kernel<D, 8><<<g, b, 0, s>>>(part, nwg, out, odt);
    else
        attn_merge_kernel<D, kAttnMaxWG / kMergeRows><<<g, b, 0, s>>>(part, nwg, out, odt);
}

size_t attn_workspace_bytes(int T, int D) {
    const int tiles = (T + kAttnTile - 1) / kAttnTile;
    const int nwg = tiles < kAttnMaxWG ? tiles : kAttnMaxWG;
    return (size_t)nwg * (size_t)(32 + kAttnHeads * D) * sizeof(float);
}

int launch_attn_decode(const uint16_t* q, const uint16_t* K, int ldk, const uint16_t* Vt,
                       const int32_t* pos, int T, int D, int cur, int window, float scale,
                       void* ws, void* out, int odt, hipStream_t s) {
    AttnArgs a;
    a.q = q;
    a.K = K;
    a.Vt = Vt;
    a.pos = pos;
    a.part = static_cast<float*>(ws);
    a.ldk = ldk;
    a.T = T;
    a.cur = cur;
    a.window = window;
    a.tiles = (T + kAttnTile - 1) / kAttnTile;
    a.nwg = a.tiles < kAttnMaxWG ? a.tiles : kAttnMaxWG;
    a.scale2 = scale * kLog2e;
    const dim3 g(a.nwg), b(256);
    if (D == 512) {
        if (pos)
            attn_split_kernel<512, true><<<g, b, 0, s>>>(a);
        else
            attn_split_kernel<512, false><<<g, b, 0, s>>>(a);
        launch_merge<512>(a.part, a.nwg, out, odt, s);
    } else {
        if (pos)
            attn_split_kernel<256, true><<<g, b, 0, s>>>(a);
        else
            attn_split_kernel<256, false><<<g, b, 0, s>>>(a);
        launch_merge<256>(a.part, a.nwg, out, odt, s);
    }
    return hip_fail(hipGetLastError(), "attention launch");
}

int launch_attn_pack_v(const uint16_t* V, int ldv, int T, int D, uint16_t* Vt, hipStream_t s) {
    const long long rows = (long long)((T + kAttnTile - 1) / kAttnTile) * D;
    attn_pack_v_kernel<<<dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s>>>(V, ldv, T, D, Vt);
    return hip_fail(hipGetLastError(), "attention V pack launch");
}

int launch_attn_store_kv(const uint16_t* k, const uint16_t* v, int slot, uint16_t* K, int ldk,
                         uint16_t* Vt, int D, hipStream_t s) {
    attn_store_kv_kernel<<<dim3(1), dim3(256), 0, s>>>(k, v, slot, K, ldk, Vt, D);
    return hip_fail(hipGetLastError(), "attention cache store launch");
}

}  // namespace w4
