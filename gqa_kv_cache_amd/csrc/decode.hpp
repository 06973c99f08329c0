// GQA decode kernels for gfx950.
//
// One workgroup per (sequence b, KV head g, split s) streams rows
// [s*chunk, min((s+1)*chunk, seqlens[b])) of K and V for head g once and
// serves every query head of the group from them ("GQA reading notes",
// zhongzhuzhou.org, walkthrough of Algorithm 2: fuse the group's queries so
// each cached K vector is read once).  Each split keeps a running maximum m,
// a running sum of weights l and an unnormalised weighted sum acc (online
// softmax).  With one split the workgroup writes the output; otherwise it
// writes (m, l, acc) to the workspace and decode_merge combines the splits
// (the long sequence cut into blocks computed independently and then fused:
// "GQA注意力机制" article, intelliparadigm.com, section 4.2).
//
// Softmax runs in base 2: scores are multiplied by scale*log2(e) and the
// weights are 2^(s - m), equal to e^(scale*dot - max) in exact arithmetic.
#pragma once

#include "common.hpp"

namespace gqa {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kDecodeStep = 32;  // keys one wave consumes per step (bf16 kernel)

// Raw buffer resources: a load at a byte offset at or beyond the resource's
// size returns zero without touching memory, so rows past seqlens[b] are
// never read and need no branch.
constexpr int kRawBufferWord3 = 0x00020000;  // 32-bit raw data format (gfx9 family)
constexpr int kStreamLoad = 2;               // cache policy "nt": data used once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kRawBufferWord3);
}

template <int D> struct DecodeShape {
    static constexpr int KI = D / 32;     // 32-wide head-dim slices of the score MFMA
    static constexpr int EPL = D / 16;    // head-dim values per lane in a V fragment and in O
    static constexpr int CPR = D / 8;     // 16-byte chunks per cached row
    static constexpr int RPI = 64 / CPR;  // rows covered by one row-pattern K load
    static constexpr int KLD = 32 / RPI;  // K loads per 32-key step
};

template <int D> struct VFragT;
template <> struct VFragT<128> { typedef u32x4 T; };
template <> struct VFragT<64> { typedef u32x2 T; };

// POL is the cache policy of the loads: kStreamLoad when each row is read
// once, 0 (cached) when several waves read the same rows.
template <int D, int POL>
__device__ __forceinline__ typename VFragT<D>::T load_vfrag(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (D == 128) return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL);
    else return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL);
}

// One 32-key step of one wave, as loaded: K rows (row pattern: each load
// covers RPI whole rows) and V rows (each load covers 4 whole rows).
template <int D> struct DecodeStepData {
    u32x4 kR[DecodeShape<D>::KLD];
    typename VFragT<D>::T vB[2][4];
};

template <int D, int POL = kStreamLoad>
__device__ __forceinline__ void decode_load_step(DecodeStepData<D>& st, __amdgpu_buffer_rsrc_t kr,
                                                 __amdgpu_buffer_rsrc_t vr, int rs2, int key0,
                                                 int lane) {
    typedef DecodeShape<D> Sh;
    const int col = lane & 15, grp = lane >> 4;
    const int vk = (key0 + lane / Sh::CPR) * rs2 + 16 * (lane % Sh::CPR);
#pragma unroll
    for (int i = 0; i < Sh::KLD; ++i)
        st.kR[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, vk, Sh::RPI * i * rs2, POL);
    const int vv = (key0 + 4 * grp) * rs2 + 2 * Sh::EPL * col;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.vB[t][r] = load_vfrag<D, POL>(vr, vv, (16 * t + r) * rs2);
}

// Consume one step: K rows go through the wave's LDS tile (XOR-swizzled by
// row so both the row-pattern writes and the MFMA-layout reads are free of
// bank conflicts), then scores, online softmax and P*V on the matrix cores.
template <int D, int NT>
__device__ __forceinline__ void decode_compute_step(const DecodeStepData<D>& st, u32x4* kt, int key0,
                                                    int end, int lane, float c_log2,
                                                    const bf16x8 (&qB)[NT][DecodeShape<D>::KI],
                                                    f32x4 (&O)[NT][DecodeShape<D>::EPL],
                                                    float (&m_run)[NT], float (&l_run)[NT]) {
    typedef DecodeShape<D> Sh;
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < Sh::KLD; ++i) {
        const int kl = Sh::RPI * i + lane / Sh::CPR;
        kt[kl * Sh::CPR + ((lane % Sh::CPR) ^ (kl % Sh::CPR))] = st.kR[i];
    }
    u32x4 kA[2][Sh::KI];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < Sh::KI; ++i) {
            const int kl = 16 * t + col;
            kA[t][i] = kt[kl * Sh::CPR + ((4 * i + grp) ^ (kl % Sh::CPR))];
        }

    // V fragments for the P*V product: element 4t+r of lane (col, grp) is
    // V[key0 + 16t + 4grp + r][EPL*col + e].
    u32x4 vT[Sh::EPL];
#pragma unroll
    for (int e = 0; e < Sh::EPL; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = j >> 1, r = 2 * (j & 1);
            const uint32_t w0 = st.vB[t][r][e >> 1];
            const uint32_t w1 = st.vB[t][r + 1][e >> 1];
            vT[e][j] = (e & 1) ? pack_hi16(w0, w1) : pack_lo16(w0, w1);
        }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float p[8];
        float mx = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < Sh::KI; ++i) acc = mfma16x16x32(as_bf16x8(kA[t][i]), qB[nt][i], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * t + 4 * grp + r;
                const float sv = key < end ? acc[r] * c_log2 : kNegInf;
                p[4 * t + r] = sv;
                mx = fmaxf(mx, sv);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[nt], mx);
        const float alpha = fast_exp2(m_run[nt] - m_new);
        m_run[nt] = m_new;
        float psum = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            p[x] = fast_exp2(p[x] - m_new);
            psum += p[x];
        }
        l_run[nt] = l_run[nt] * alpha + psum;

        // Rescale O: its rows are heads 16nt + 4grp + r, whose alpha sits in lane 4grp + r.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
            for (int e = 0; e < Sh::EPL; ++e) O[nt][e][r] *= ar;
        }

        u32x4 phi, plo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = __float_as_uint(p[2 * j]);
            const uint32_t c = __float_as_uint(p[2 * j + 1]);
            phi[j] = pack_hi16(a, c);
            const float al = p[2 * j] - __uint_as_float(a & 0xffff0000u);
            const float cl = p[2 * j + 1] - __uint_as_float(c & 0xffff0000u);
            plo[j] = pack_bf16x2_rne(al, cl);
        }
#pragma unroll
        for (int e = 0; e < Sh::EPL; ++e) {
            O[nt][e] = mfma16x16x32(as_bf16x8(phi), as_bf16x8(vT[e]), O[nt][e]);
            O[nt][e] = mfma16x16x32(as_bf16x8(plo), as_bf16x8(vT[e]), O[nt][e]);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 split kernel on the matrix cores.
//
// Per wave and step of 32 keys (two 16-key sub-tiles t):
//   loads   K and V rows are streamed with whole-row ("row pattern") loads
//           that bypass cache allocation; K is rearranged through LDS.
//   scores  S^T[key][head] = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows
//           (lane: key 16t + lane%16, 8 head-dim values), B = the group's
//           queries (lane: head lane%16, same 8 head-dim values); the 16
//           MFMA columns are up to 16 query heads of the group, so one K
//           fragment serves them all.  Products of bf16 values are exact in
//           fp32 and the sum is fp32.
//   result  lane holds the scores of keys 16t + 4*(lane/16) + r (r < 4) for
//           head lane%16 -- exactly the A-operand layout of the P*V product.
//   P*V     O[head][dim] += P[head][key] V[key][dim], again 16x16x32 MFMA;
//           V fragments are 8 keys x 1 head-dim value per lane, built from
//           the row loads with byte permutes.  P is fed as two bf16 terms,
//           hi = truncation of p and lo = p - hi rounded, so the weights
//           carry ~16 significant bits and the accumulation is fp32.
// NT = number of 16-head tiles (ceil(group size / 16)).
// ---------------------------------------------------------------------------
template <int D, int NT>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ seqlens, int Hq, int Hkv,
    int Lmax, int gsize, int S, int chunk, float c_log2, uint16_t* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
    typedef DecodeShape<D> Sh;
    constexpr int KI = Sh::KI;
    constexpr int EPL = Sh::EPL;

    __shared__ float sm_m[16 * kDecodeWaves];  // per wave: running max of each head of a tile
    __shared__ float sm_l[16 * kDecodeWaves];  // per wave: weight sum of each head of a tile
    __shared__ u32x4 k_tiles[kDecodeWaves][32 * Sh::CPR];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    // (b, KV head) varies fastest and the piece slowest: workgroups are dealt
    // to the XCDs round-robin, so each XCD gets the same mix of pieces, and
    // every first piece (always full) is dispatched before any later one.
    const int nbg = gridDim.x / S;
    const int s = blockIdx.x / nbg;
    const int bg = blockIdx.x % nbg;
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int n = valid_rows(seqlens[b], Lmax);
    const int start = s * chunk;
    const int end = min(start + chunk, n);
    if (S > 1 && start >= end) return;  // empty split: the merge skips it

    const int rs2 = Hkv * D * 2;  // bytes between consecutive keys of one head
    const uint16_t* kb = kc + ((int64_t)b * Lmax * Hkv + g) * D;
    const uint16_t* vb = vc + ((int64_t)b * Lmax * Hkv + g) * D;
    const int valid_bytes = end > 0 ? (end - 1) * rs2 + D * 2 : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, valid_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, valid_bytes);
    u32x4* kt = k_tiles[wave];
    const int h0 = g * gsize;

    bf16x8 qB[NT][KI];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int hq = 16 * nt + col;
        const bool ok = hq < gsize;
        const uint16_t* qp = q + ((int64_t)b * Hq + h0 + (ok ? hq : 0)) * D + 8 * grp;
#pragma unroll
        for (int i = 0; i < KI; ++i) qB[nt][i] = as_bf16x8(load16(qp + 32 * i, ok));
    }

    f32x4 O[NT][EPL];
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = kNegInf;
        l_run[nt] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) O[nt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The next step's rows are requested before this step is computed, so a
    // wave's loads overlap its own compute.
    constexpr int stride = kDecodeWaves * kDecodeStep;
    int key0 = start + wave * kDecodeStep;
    DecodeStepData<D> cur;
    if (key0 < end) decode_load_step<D>(cur, kr, vr, rs2, key0, lane);
    for (; key0 < end; key0 += stride) {
        DecodeStepData<D> nxt;
        if (key0 + stride < end) decode_load_step<D>(nxt, kr, vr, rs2, key0 + stride, lane);
        decode_compute_step<D, NT>(cur, kt, key0, end, lane, c_log2, qB, O, m_run, l_run);
        cur = nxt;
    }

    // Sum of weights across the four lane groups that share a head.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        l_run[nt] += __shfl_xor(l_run[nt], 16);
        l_run[nt] += __shfl_xor(l_run[nt], 32);
    }

    // Combine the waves' partial results, one 16-head tile at a time: each
    // wave's part of the tile (16 heads x D floats) is staged in its own K
    // tile, which it no longer reads, and after a barrier every thread
    // combines one (head, 8 head-dim values) piece over the four waves.
    float* part = reinterpret_cast<float*>(kt);
    static_assert(16 * D * sizeof(float) <= 32 * Sh::CPR * sizeof(u32x4), "a tile's part fits the K tile");
    constexpr int C8 = D / 8;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (nt > 0) __syncthreads();  // the previous tile's parts have been read
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * grp + r;
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
                *reinterpret_cast<f32x4*>(part + h * D + EPL * col + e) =
                    f32x4{O[nt][e][r], O[nt][e + 1][r], O[nt][e + 2][r], O[nt][e + 3][r]};
        }
        if (grp == 0) {
            sm_m[wave * 16 + col] = m_run[nt];
            sm_l[wave * 16 + col] = l_run[nt];
        }
        __syncthreads();
        const int items = min(16, gsize - 16 * nt) * C8;
        for (int it = threadIdx.x; it < items; it += kDecodeThreads) {
            const int i = it / C8;
            const int c = (it % C8) * 8;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w * 16 + i]);
            float L = 0.f;
            f32x4 o0 = f32x4{0.f, 0.f, 0.f, 0.f}, o1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) {
                const float f = M == kNegInf ? 0.f : fast_exp2(sm_m[w * 16 + i] - M);
                L += f * sm_l[w * 16 + i];
                const float* src = reinterpret_cast<const float*>(k_tiles[w]) + i * D + c;
                o0 += f * *reinterpret_cast<const f32x4*>(src);
                o1 += f * *reinterpret_cast<const f32x4*>(src + 4);
            }
            const int64_t row = (int64_t)b * Hq + h0 + 16 * nt + i;
            if (S == 1) {
                const float inv = L > 0.f ? 1.f / L : 0.f;
                u32x4 o;
                o[0] = pack_bf16x2_rne(o0[0] * inv, o0[1] * inv);
                o[1] = pack_bf16x2_rne(o0[2] * inv, o0[3] * inv);
                o[2] = pack_bf16x2_rne(o1[0] * inv, o1[1] * inv);
                o[3] = pack_bf16x2_rne(o1[2] * inv, o1[3] * inv);
                *reinterpret_cast<u32x4*>(out + row * D + c) = o;
            } else {
                float* dst = ws_acc + (row * S + s) * D + c;
                *reinterpret_cast<f32x4*>(dst) = o0;
                *reinterpret_cast<f32x4*>(dst + 4) = o1;
                if (c == 0) {
                    ws_ml[(row * S + s) * 2] = M;
                    ws_ml[(row * S + s) * 2 + 1] = L;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 split kernel for groups of 49..64 query heads (four 16-head tiles).
//
// Each of the four waves owns one tile of heads and streams every row of the
// piece itself, with the same step as decode_split_bf16, so no partial
// results are combined across waves.  The four waves read the same rows at
// about the same time; their loads go through L2 (default cache policy),
// which serves the repeats, so memory still supplies each row once.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_bf16_tiles(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ seqlens, int Hq, int Hkv,
    int Lmax, int gsize, int S, int chunk, float c_log2, uint16_t* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
    typedef DecodeShape<D> Sh;
    constexpr int KI = Sh::KI;
    constexpr int EPL = Sh::EPL;
    static_assert(kDecodeWaves == 4, "one 16-head tile per wave");

    __shared__ u32x4 k_tiles[kDecodeWaves][32 * Sh::CPR];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int nbg = gridDim.x / S;
    const int s = blockIdx.x / nbg;
    const int bg = blockIdx.x % nbg;
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int n = valid_rows(seqlens[b], Lmax);
    const int start = s * chunk;
    const int end = min(start + chunk, n);
    if (S > 1 && start >= end) return;  // empty split: the merge skips it

    const int rs2 = Hkv * D * 2;
    const uint16_t* kb = kc + ((int64_t)b * Lmax * Hkv + g) * D;
    const uint16_t* vb = vc + ((int64_t)b * Lmax * Hkv + g) * D;
    const int valid_bytes = end > 0 ? (end - 1) * rs2 + D * 2 : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, valid_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, valid_bytes);
    u32x4* kt = k_tiles[wave];
    const int h0 = g * gsize;
    const int ht = 16 * wave;  // first head of this wave's tile, within the group

    bf16x8 qB[1][KI];
    {
        const int hq = ht + col;
        const bool ok = hq < gsize;
        const uint16_t* qp = q + ((int64_t)b * Hq + h0 + (ok ? hq : 0)) * D + 8 * grp;
#pragma unroll
        for (int i = 0; i < KI; ++i) qB[0][i] = as_bf16x8(load16(qp + 32 * i, ok));
    }
    f32x4 O[1][EPL];
    float m_run[1] = {kNegInf}, l_run[1] = {0.f};
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[0][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    int key0 = start;
    DecodeStepData<D> cur;
    if (key0 < end) decode_load_step<D, 0>(cur, kr, vr, rs2, key0, lane);
    for (; key0 < end; key0 += kDecodeStep) {
        DecodeStepData<D> nxt;
        if (key0 + kDecodeStep < end) decode_load_step<D, 0>(nxt, kr, vr, rs2, key0 + kDecodeStep, lane);
        decode_compute_step<D, 1>(cur, kt, key0, end, lane, c_log2, qB, O, m_run, l_run);
        cur = nxt;
    }

    // Sum of weights across the four lane groups that share a head (lane col
    // holds head ht + col); O row r of lane (col, grp) is head ht + 4grp + r.
    float l = l_run[0];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float lr[4], mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        lr[r] = __shfl(l, 4 * grp + r);
        mr[r] = __shfl(m_run[0], 4 * grp + r);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = ht + 4 * grp + r;
        if (h >= gsize) continue;
        const int64_t row = (int64_t)b * Hq + h0 + h;
        if (S == 1) {
            u32x4 o;
#pragma unroll
            for (int j = 0; j < EPL / 2; ++j) {
                const float x0 = lr[r] > 0.f ? O[0][2 * j][r] / lr[r] : 0.f;
                const float x1 = lr[r] > 0.f ? O[0][2 * j + 1][r] / lr[r] : 0.f;
                o[j] = pack_bf16x2_rne(x0, x1);
            }
            uint16_t* dst = out + row * D + EPL * col;
            if constexpr (EPL == 8) *reinterpret_cast<u32x4*>(dst) = o;
            else *reinterpret_cast<u32x2*>(dst) = u32x2{o[0], o[1]};
        } else {
            float* dst = ws_acc + (row * S + s) * D + EPL * col;
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
                *reinterpret_cast<f32x4*>(dst + e) = f32x4{O[0][e][r], O[0][e + 1][r], O[0][e + 2][r], O[0][e + 3][r]};
            if (col == 0) {
                ws_ml[(row * S + s) * 2] = mr[r];
                ws_ml[(row * S + s) * 2 + 1] = lr[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 split kernel on the vector ALUs (fp32 inputs).
//
// Per tile of 64 keys: the tile's K and V rows, fetched into registers with
// coalesced 16-byte loads while the previous tile was being computed (rows
// at or past the piece end are never read), are staged in LDS; scores for
// every (head of the group, key) pair go to LDS; one wave per head updates
// that head's online softmax (one key per lane, shuffle reductions); then
// each thread accumulates its (head, head-dim) outputs over the tile.  The
// query is staged in LDS already multiplied by scale*log2(e).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_f32(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ seqlens, int Hq, int Hkv, int Lmax, int gsize, int S, int chunk,
    float c_log2, float* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
    constexpr int TILE = 64;   // keys per tile: one per lane in the softmax
    constexpr int MAXG = 64;
    constexpr int ACC = MAXG * D / kDecodeThreads;
    constexpr int RP = D + 4;  // padded LDS row: rows 4 banks apart for the score reads
    constexpr int C4 = D / 4;  // 16-byte pieces per row
    constexpr int PER = TILE * C4 / kDecodeThreads;  // pieces per thread and operand

    __shared__ float sq[MAXG * D];
    __shared__ float ss[MAXG * TILE];
    __shared__ __align__(16) float sk[TILE * RP];
    __shared__ __align__(16) float sv[TILE * D];
    __shared__ float sm[MAXG], sl[MAXG], sa[MAXG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // (b, KV head) varies fastest and the piece slowest: workgroups are dealt
    // to the XCDs round-robin, so each XCD gets the same mix of pieces, and
    // every first piece (always full) is dispatched before any later one.
    const int nbg = gridDim.x / S;
    const int s = blockIdx.x / nbg;
    const int bg = blockIdx.x % nbg;
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int n = valid_rows(seqlens[b], Lmax);
    const int start = s * chunk;
    const int end = min(start + chunk, n);
    if (S > 1 && start >= end) return;
    const int h0 = g * gsize;
    const int64_t rs = (int64_t)Hkv * D;
    const float* kb = kc + ((int64_t)b * Lmax * Hkv + g) * D;
    const float* vb = vc + ((int64_t)b * Lmax * Hkv + g) * D;

    for (int idx = tid; idx < gsize * D; idx += kDecodeThreads)
        sq[idx] = q[((int64_t)b * Hq + h0) * D + idx] * c_log2;
    for (int h = tid; h < gsize; h += kDecodeThreads) {
        sm[h] = kNegInf;
        sl[h] = 0.f;
    }
    float acc[ACC];
#pragma unroll
    for (int i = 0; i < ACC; ++i) acc[i] = 0.f;

    f32x4 nk[PER], nv[PER];
    auto fetch = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = tid + kDecodeThreads * p;
            const int j = idx / C4, c = 4 * (idx % C4);
            nk[p] = nv[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t0 + j < end) {
                nk[p] = *reinterpret_cast<const f32x4*>(kb + (int64_t)(t0 + j) * rs + c);
                nv[p] = *reinterpret_cast<const f32x4*>(vb + (int64_t)(t0 + j) * rs + c);
            }
        }
    };
    if (start < end) fetch(start);
    for (int t0 = start; t0 < end; t0 += TILE) {
        const int cnt = min(TILE, end - t0);
        __syncthreads();  // the previous tile's K, V and scores have been read
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = tid + kDecodeThreads * p;
            const int j = idx / C4, c = 4 * (idx % C4);
            *reinterpret_cast<f32x4*>(sk + j * RP + c) = nk[p];
            *reinterpret_cast<f32x4*>(sv + j * D + c) = nv[p];
        }
        __syncthreads();
        if (t0 + TILE < end) fetch(t0 + TILE);  // in flight while this tile is computed
        for (int idx = tid; idx < gsize * TILE; idx += kDecodeThreads) {
            const int h = idx / TILE, j = idx % TILE;
            float sc = kNegInf;
            if (j < cnt) {
                const float* qh = sq + h * D;
                const float* kr = sk + j * RP;
                float dot = 0.f;
                for (int c = 0; c < D; ++c) dot += qh[c] * kr[c];
                sc = dot;
            }
            ss[h * TILE + j] = sc;
        }
        __syncthreads();
        for (int h = wave; h < gsize; h += kDecodeWaves) {
            const float sc = ss[h * TILE + lane];  // -inf past cnt
            float mx = sc;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float mo = sm[h];
            const float mn = fmaxf(mo, mx);
            const float pj = fast_exp2(sc - mn);
            float sum = pj;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
            ss[h * TILE + lane] = pj;
            if (lane == 0) {
                const float a = fast_exp2(mo - mn);
                sl[h] = sl[h] * a + sum;
                sm[h] = mn;
                sa[h] = a;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ACC; ++i) {
            const int idx = tid + kDecodeThreads * i;
            if (idx < gsize * D) {
                const int h = idx / D, c = idx % D;
                float a = acc[i] * sa[h];
                for (int j = 0; j < cnt; ++j) a += ss[h * TILE + j] * sv[j * D + c];
                acc[i] = a;
            }
        }
    }
    __syncthreads();  // sm, sl are complete (also when the piece is empty)

#pragma unroll
    for (int i = 0; i < ACC; ++i) {
        const int idx = tid + kDecodeThreads * i;
        if (idx < gsize * D) {
            const int h = idx / D, c = idx % D;
            const int64_t row = (int64_t)b * Hq + h0 + h;
            if (S == 1) {
                out[row * D + c] = sl[h] > 0.f ? acc[i] / sl[h] : 0.f;
            } else {
                ws_acc[(row * S + s) * D + c] = acc[i];
                if (c == 0) {
                    ws_ml[(row * S + s) * 2] = sm[h];
                    ws_ml[(row * S + s) * 2 + 1] = sl[h];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of the split partials: M = max_s m_s, out = sum_s 2^(m_s-M) acc_s /
// sum_s 2^(m_s-M) l_s over the splits s in [s0, se) that hold keys of the
// row (the plain decode: s0 = 0, se = ceil(seqlens[b]/chunk)).  One 64-lane
// wave per row.  Lane i holds the (m, l) of split g0 + i of the current group
// of 64 splits; every lane holds its D/64 columns of each split.  The row's
// length, the first group's (m, l) pairs and the first 16 splits' columns
// are all requested before the split range is known, so a row of up to 16
// splits waits on memory once instead of once per split.  Slots outside the
// range are never used (a select, not a multiply by 0, so stale workspace
// contents cannot leak in).
// ---------------------------------------------------------------------------
constexpr int kMergeChunk = 16;  // splits whose columns are requested at once

template <int D, typename Range>
__device__ __forceinline__ float merge_split_row(const float* __restrict__ ws_acc,
                                                 const float* __restrict__ ws_ml, int n,
                                                 int64_t row, int S, Range range,
                                                 float (&acc)[D / 64]) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const float* arow = ws_acc + row * S * D + lane * PER;
    const float* mrow = ws_ml + row * S * 2;
    float m0 = kNegInf, l0 = 0.f;
    if (lane < S) {
        const float2 v = *reinterpret_cast<const float2*>(mrow + 2 * lane);
        m0 = v.x;
        l0 = v.y;
    }
    float a[kMergeChunk][PER];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
        if (i < S) {
            if constexpr (PER == 2) {
                const float2 v = *reinterpret_cast<const float2*>(arow + i * D);
                a[i][0] = v.x;
                a[i][PER - 1] = v.y;
            } else {
                a[i][0] = arow[i * D];
            }
        }
    }
    int s0, se;
    range(n, s0, se);
    // M over every split in range (further groups only when S > 64)
    float M = (lane >= s0 && lane < se && m0 != kNegInf) ? m0 : kNegInf;
    for (int g0 = 64; g0 < se; g0 += 64) {
        const int sl = g0 + lane;
        if (sl >= s0 && sl < se) {
            const float m = mrow[2 * sl];
            if (m != kNegInf) M = fmaxf(M, m);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] = 0.f;
    float L = 0.f;
    for (int g0 = 0; g0 < se; g0 += 64) {
        float m = m0, l = l0;
        const int sl = g0 + lane;
        if (g0 > 0) {
            m = kNegInf;
            l = 0.f;
            if (sl < se) {
                m = mrow[2 * sl];
                l = mrow[2 * sl + 1];
            }
        }
        const bool mine = sl >= s0 && sl < se && m != kNegInf;
        const float f = mine ? fast_exp2(m - M) : 0.f;
        if (mine) L += f * l;
        const int gend = min(se, g0 + 64);
        for (int base = g0; base < gend; base += kMergeChunk) {
            if (base > 0) {
#pragma unroll
                for (int i = 0; i < kMergeChunk; ++i) {
                    if (base + i < gend) {
#pragma unroll
                        for (int p = 0; p < PER; ++p) a[i][p] = arow[(base + i) * D + p];
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < kMergeChunk; ++i) {
                const int s = base + i;
                if (s >= s0 && s < gend) {
                    const float fs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), s - g0));
#pragma unroll
                    for (int p = 0; p < PER; ++p) acc[p] += fs * a[i][p];
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    return L;
}

template <int D, bool BF16OUT>
__global__ __launch_bounds__(64) void decode_merge(const float* __restrict__ ws_acc,
                                                   const float* __restrict__ ws_ml,
                                                   const int32_t* __restrict__ seqlens, int Hq,
                                                   int Lmax, int S, int chunk,
                                                   void* __restrict__ out) {
    constexpr int PER = D / 64;
    const int64_t row = blockIdx.x;
    const int n = valid_rows(seqlens[row / Hq], Lmax);
    float acc[PER];
    const float L = merge_split_row<D>(ws_acc, ws_ml, n, row, S, [&](int len, int& s0, int& se) {
        s0 = 0;
        se = min(S, (len + chunk - 1) / chunk);
    }, acc);
    const int c0 = threadIdx.x * PER;
    float o[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) o[p] = L > 0.f ? acc[p] / L : 0.f;
    if (BF16OUT) {
        uint16_t* dst = static_cast<uint16_t*>(out) + row * D + c0;
        if (PER == 2)
            *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2_rne(o[0], o[PER - 1]);
        else
            dst[0] = (uint16_t)f32_to_bf16_rne(o[0]);
    } else {
        float* dst = static_cast<float*>(out) + row * D + c0;
#pragma unroll
        for (int p = 0; p < PER; ++p) dst[p] = o[p];
    }
}

}  // namespace gqa
