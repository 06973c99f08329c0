// Extended GQA decode for gfx950: several new query tokens per sequence, an
// optional sliding window, a paged cache and an FP8 (OCP E4M3 or E5M2) cache.
//
// Same structure as the plain decode kernel (one workgroup per sequence, KV
// head and split; whole-row loads; K rearranged through a per-wave LDS tile;
// scores and P*V on v_mfma_f32_16x16x32_bf16), generalised:
//   - The workgroup's query rows are (token, head) pairs of the group, row
//     r = t * gsize + h', up to 64 of them.  Token t of a sequence with n
//     valid rows sits at position n - T + t and sees keys
//     [max(0, pos - W + 1), pos] (W = window, 0 = all): causal among the new
//     tokens as in prefill ("从MHA到GQA", causal mask section), restricted to
//     a window when one is given.
//   - Each 16-row half of a wave's 32-key step gets its own buffer resource
//     based at the half's first row: in a paged cache that row lives in
//     block block_table[b][row / block_size] (block_size a multiple of 16,
//     so a half never crosses a block; the two halves may lie in different
//     blocks).  A resource's size ends at the last valid row, so rows at or
//     past the split end read as zero.
//   - FP8 rows are converted to bf16 (exact: every E4M3 and every E5M2 value
//     is a bf16 value) when K is staged in LDS and when the V fragments are built.  The
//     per-KV-head scales never touch the elements: k_scale multiplies the
//     score factor and v_scale the output.
//   - The append of the T new rows (Algorithm 2 of "GQA reading notes" stores
//     the new K/V before attending) happens in the same launch: rows at or
//     past n - T are read from k_new/v_new instead of the cache, and the
//     workgroup whose piece holds such a row stores it into the cache.  No
//     workgroup reads a cache row that another one writes in the same call.
// Splits write (m, l, acc) like the plain kernel; decode_ex_merge combines
// the splits that intersect the keys any token of the sequence can see.
#pragma once

#include "common.hpp"
#include "decode.hpp"

namespace gqa {

// Byte-level geometry of one cached row.
template <int D, bool KV8> struct ExShape {
    static constexpr int ELT = KV8 ? 1 : 2;            // bytes per stored element
    static constexpr int ROWB = D * ELT;               // bytes per row of one KV head
    static constexpr int CPR = ROWB / 16;              // 16-byte chunks per stored row
    static constexpr int RPI = 64 / CPR;               // rows per whole-row K load
    static constexpr int KLD = 32 / RPI;               // K loads per 32-key step
    static constexpr int VB = DecodeShape<D>::EPL * ELT;  // bytes of one lane's V piece per row
};

// Raw V piece of one row for one lane: EPL elements.
template <int D, bool KV8> struct ExVRaw;
template <> struct ExVRaw<128, false> { typedef u32x4 T; };
template <> struct ExVRaw<64, false> { typedef u32x2 T; };
template <> struct ExVRaw<128, true> { typedef u32x2 T; };
template <> struct ExVRaw<64, true> { typedef uint32_t T; };

template <int D, bool KV8>
__device__ __forceinline__ typename ExVRaw<D, KV8>::T ex_load_v(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (ExShape<D, KV8>::VB == 16) return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamLoad);
    else if constexpr (ExShape<D, KV8>::VB == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamLoad);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamLoad);
}

// Two FP8 bytes (low or high half of a word) -> two bf16 in one word; KV is
// the cache format: 1 = E4M3, 2 = E5M2.
template <int KV, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    if constexpr (KV == 2) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
    else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// V piece as bf16 words (the plain kernel's VFragT layout).
template <int D, int KV>
__device__ __forceinline__ typename VFragT<D>::T ex_v_bf16(typename ExVRaw<D, KV != 0>::T x) {
    if constexpr (KV == 0) {
        return x;
    } else if constexpr (D == 128) {
        return u32x4{fp8x2_to_bf16x2<KV, false>(x[0]), fp8x2_to_bf16x2<KV, true>(x[0]),
                     fp8x2_to_bf16x2<KV, false>(x[1]), fp8x2_to_bf16x2<KV, true>(x[1])};
    } else {
        return u32x2{fp8x2_to_bf16x2<KV, false>(x), fp8x2_to_bf16x2<KV, true>(x)};
    }
}

template <int D, bool KV8> struct ExStepData {
    u32x4 kR[ExShape<D, KV8>::KLD];
    typename ExVRaw<D, KV8>::T vB[2][4];
};

// Loads of one 32-key step.  kr[x], vr[x] cover rows 16x .. 16x+15 of the
// step.  H16: two resources, each based at its half's first row (the halves
// may lie in different cache blocks); otherwise one resource for the whole
// step (both entries equal).  A whole-row K load covers RPI rows (4, 8 or
// 16, a divisor of 16), so it stays in one half.
template <int D, bool KV8, bool H16>
__device__ __forceinline__ void ex_load_step(ExStepData<D, KV8>& st, const __amdgpu_buffer_rsrc_t (&kr)[2],
                                             const __amdgpu_buffer_rsrc_t (&vr)[2], int rs, int lane) {
    typedef ExShape<D, KV8> Sh;
    static_assert(16 % Sh::RPI == 0, "a K load must not straddle the two halves of a step");
    const int col = lane & 15, grp = lane >> 4;
    const int vk = (lane / Sh::CPR) * rs + 16 * (lane % Sh::CPR);
#pragma unroll
    for (int i = 0; i < Sh::KLD; ++i) {
        const int row = Sh::RPI * i;  // first row of this load within the step
        if constexpr (H16)
            st.kR[i] = __builtin_amdgcn_raw_buffer_load_b128(kr[row / 16], vk, (row % 16) * rs, kStreamLoad);
        else
            st.kR[i] = __builtin_amdgcn_raw_buffer_load_b128(kr[0], vk, row * rs, kStreamLoad);
    }
    const int vv = 4 * grp * rs + Sh::VB * col;  // rows r + 4 grp of a half, r < 4
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (H16)
                st.vB[t][r] = ex_load_v<D, KV8>(vr[t], vv, r * rs);
            else
                st.vB[t][r] = ex_load_v<D, KV8>(vr[0], vv, (16 * t + r) * rs);
        }
}

// The rows of a step at or past `nw` (the first appended row) come from the
// new rows [B,T,Hkv,d] instead of the cache, whose resource ends before them
// and so returned zeros there: OR the new rows in.  Rows at or past `end`
// stay zero.  kn/vn point at new row (b, 0, g).
template <int D, bool KV8>
__device__ __forceinline__ void ex_merge_new_rows(ExStepData<D, KV8>& st, const uint8_t* kn,
                                                  const uint8_t* vn, int key0, int nw, int end,
                                                  int T, int rs, int lane) {
    typedef ExShape<D, KV8> Sh;
    typedef typename ExVRaw<D, KV8>::T VR;
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < Sh::KLD; ++i) {
        const int row = key0 + Sh::RPI * i + lane / Sh::CPR;
        const int t = row - nw;
        if (t >= 0 && t < T && row < end)
            st.kR[i] |= *reinterpret_cast<const u32x4*>(kn + (int64_t)t * rs + 16 * (lane % Sh::CPR));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = key0 + 16 * h + 4 * grp + r;
            const int t = row - nw;
            if (t >= 0 && t < T && row < end)
                st.vB[h][r] |= *reinterpret_cast<const VR*>(vn + (int64_t)t * rs + Sh::VB * col);
        }
}

// K rows into the wave's LDS tile as bf16, in the plain kernel's swizzled
// layout (row kl, 16-byte bf16 chunk c at kl*CPR + (c ^ (kl % CPR))).
template <int D, int KV>
__device__ __forceinline__ void ex_stage_k(const ExStepData<D, KV != 0>& st, u32x4* kt, int lane) {
    constexpr bool KV8 = KV != 0;
    typedef ExShape<D, KV8> Sh;
    constexpr int CPR16 = DecodeShape<D>::CPR;  // bf16 chunks per row
#pragma unroll
    for (int i = 0; i < Sh::KLD; ++i) {
        const int kl = Sh::RPI * i + lane / Sh::CPR;
        const int c = lane % Sh::CPR;
        if constexpr (!KV8) {
            kt[kl * CPR16 + (c ^ (kl % CPR16))] = st.kR[i];
        } else {
            // 16 FP8 values = head dims 16c .. 16c+15 = bf16 chunks 2c, 2c+1
            const u32x4 w = st.kR[i];
            const u32x4 lo = u32x4{fp8x2_to_bf16x2<KV, false>(w[0]), fp8x2_to_bf16x2<KV, true>(w[0]),
                                   fp8x2_to_bf16x2<KV, false>(w[1]), fp8x2_to_bf16x2<KV, true>(w[1])};
            const u32x4 hi = u32x4{fp8x2_to_bf16x2<KV, false>(w[2]), fp8x2_to_bf16x2<KV, true>(w[2]),
                                   fp8x2_to_bf16x2<KV, false>(w[3]), fp8x2_to_bf16x2<KV, true>(w[3])};
            kt[kl * CPR16 + ((2 * c) ^ (kl % CPR16))] = lo;
            kt[kl * CPR16 + ((2 * c + 1) ^ (kl % CPR16))] = hi;
        }
    }
}

// Scores, masked online softmax and P*V of one step.  lo/hi: inclusive key
// range of each lane's query row (per 16-row tile); end: split end.
template <int D, int NT, int KV>
__device__ __forceinline__ void ex_compute_step(const ExStepData<D, KV != 0>& st, const u32x4* kt,
                                                int key0, int end, int lane, float c_log2,
                                                const int (&lo)[NT], const int (&hi)[NT],
                                                const bf16x8 (&qB)[NT][DecodeShape<D>::KI],
                                                f32x4 (&O)[NT][DecodeShape<D>::EPL],
                                                float (&m_run)[NT], float (&l_run)[NT]) {
    typedef DecodeShape<D> Sh;
    const int col = lane & 15, grp = lane >> 4;
    u32x4 kA[2][Sh::KI];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < Sh::KI; ++i) {
            const int kl = 16 * t + col;
            kA[t][i] = kt[kl * Sh::CPR + ((4 * i + grp) ^ (kl % Sh::CPR))];
        }
    typename VFragT<D>::T vB[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) vB[t][r] = ex_v_bf16<D, KV>(st.vB[t][r]);
    // element 4t+r of lane (col, grp): V[key0 + 16t + 4grp + r][EPL*col + e]
    u32x4 vT[Sh::EPL];
#pragma unroll
    for (int e = 0; e < Sh::EPL; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = j >> 1, r = 2 * (j & 1);
            const uint32_t w0 = vB[t][r][e >> 1];
            const uint32_t w1 = vB[t][r + 1][e >> 1];
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
                const bool vis = key < end && key >= lo[nt] && key <= hi[nt];
                const float sv = vis ? acc[r] * c_log2 : kNegInf;
                p[4 * t + r] = sv;
                mx = fmaxf(mx, sv);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[nt], mx);
        // a row that has seen no visible key yet keeps m = -inf; subtract 0
        // instead so its weights are 0 rather than NaN
        const float m_sub = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[nt] - m_sub);
        m_run[nt] = m_new;
        float psum = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            p[x] = fast_exp2(p[x] - m_sub);
            psum += p[x];
        }
        l_run[nt] = l_run[nt] * alpha + psum;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
            for (int e = 0; e < Sh::EPL; ++e) O[nt][e][r] *= ar;
        }
        // weights as hi + lo bf16 terms (~16 significant bits), as in the plain kernel
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

// First key any token of a sequence with n rows can see (window W, T tokens).
__device__ __forceinline__ int ex_first_key(int n, int T, int window) {
    return window > 0 ? max(0, n - T - window + 1) : 0;
}

// ---------------------------------------------------------------------------
// Split kernel.  q [B,T,Hq,d] bf16; caches contiguous [B,Lmax,Hkv,d] or a
// paged pool [nblocks,bs,Hkv,d] (bf16 or FP8 bytes); out [B,T,Hq,d] bf16.
// NT = ceil(T * gsize / 16) tiles of 16 query rows; NWV waves per workgroup
// take the split's 32-key steps in turn.
// ---------------------------------------------------------------------------
template <int D, int NT, int KV, int NWV, bool H16>
__global__ __launch_bounds__(64 * NWV) void decode_ex_kernel(
    const uint16_t* __restrict__ q, uint8_t* kc, uint8_t* vc,
    const int32_t* __restrict__ seqlens, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    int bs, int num_blocks, const uint8_t* k_new, const uint8_t* v_new, int T, int Hq, int Hkv,
    int Lmax, int gsize, int S, int chunk, int window, float c_log2, uint16_t* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
    constexpr bool KV8 = KV != 0;  // one-byte FP8 rows (KV: 1 = E4M3, 2 = E5M2)
    typedef DecodeShape<D> Sh;
    typedef ExShape<D, KV8> Ex;
    constexpr int KI = Sh::KI;
    constexpr int EPL = Sh::EPL;

    __shared__ float sm_m[16 * NWV];  // per wave: running max of each row of a tile
    __shared__ float sm_l[16 * NWV];  // per wave: weight sum of each row of a tile
    __shared__ u32x4 k_tiles[NWV][32 * Sh::CPR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int n_in = seqlens[b];
    const int n = valid_rows(n_in, Lmax);
    const int first = ex_first_key(n, T, window);
    const int start = s * chunk;
    const int end = min(start + chunk, n);
    if (max(start, first) >= end) return;  // no token sees this split: the merge skips it

    const int rs = Hkv * Ex::ROWB;  // bytes between consecutive rows of one KV head
    // First row that comes from the new rows (none without an append).
    const int nw = k_new ? n_in - T : INT_MAX;
    const uint8_t* kn = k_new ? k_new + (((int64_t)b * T) * Hkv + g) * Ex::ROWB : nullptr;
    const uint8_t* vn = v_new ? v_new + (((int64_t)b * T) * Hkv + g) * Ex::ROWB : nullptr;
    // Cache row j of this sequence and KV head; nullptr for a block id
    // outside the pool (never dereferenced then).
    auto cache_row = [&](uint8_t* base, int j) __attribute__((always_inline)) -> uint8_t* {
        if (!block_table) return base + (((int64_t)b * Lmax + j) * Hkv + g) * Ex::ROWB;
        const int blk = block_table[(int64_t)b * max_blocks + j / bs];
        if ((unsigned)blk >= (unsigned)num_blocks) return nullptr;
        return base + (((int64_t)blk * bs + j % bs) * Hkv + g) * Ex::ROWB;
    };
    if (k_new) {
        // Store the new rows of this piece: rows [nw, nw + T) inside
        // [start, start + chunk) and inside the cache.
        const int j0 = max(max(start, nw), 0);
        const int j1 = min(min(start + chunk, nw + T), Lmax);
        for (int it = threadIdx.x; it < (j1 - j0) * Ex::CPR; it += 64 * NWV) {
            const int j = j0 + it / Ex::CPR;
            const int c = 16 * (it % Ex::CPR);
            uint8_t* kd = cache_row(kc, j);
            uint8_t* vd = cache_row(vc, j);
            if (!kd) continue;
            *reinterpret_cast<u32x4*>(kd + c) = *reinterpret_cast<const u32x4*>(kn + (int64_t)(j - nw) * rs + c);
            *reinterpret_cast<u32x4*>(vd + c) = *reinterpret_cast<const u32x4*>(vn + (int64_t)(j - nw) * rs + c);
        }
    }
    const int R = T * gsize;        // query rows of the workgroup
    const int h0 = g * gsize;
    u32x4* kt = k_tiles[wave];
    float cs = c_log2;
    if constexpr (KV8) cs *= k_scale[g];

    bf16x8 qB[NT][KI];
    int lo[NT], hi[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + col;
        const bool ok = r < R;
        const int t = ok ? r / gsize : 0, hh = ok ? r % gsize : 0;
        const uint16_t* qp = q + (((int64_t)b * T + t) * Hq + h0 + hh) * D + 8 * grp;
#pragma unroll
        for (int i = 0; i < KI; ++i) qB[nt][i] = as_bf16x8(load16(qp + 32 * i, ok));
        const int pos = n - T + t;
        hi[nt] = ok ? pos : -1;
        lo[nt] = window > 0 ? max(0, pos - window + 1) : 0;
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

    // 32-aligned first step (start is a multiple of 32; the window start may not be)
    const int kbeg = max(start, first & ~31);
    const uint8_t* kseq = kc + (((int64_t)b * Lmax) * Hkv + g) * Ex::ROWB;
    const uint8_t* vseq = vc + (((int64_t)b * Lmax) * Hkv + g) * Ex::ROWB;
    // Issue the loads of the step starting at key0, through resources sized
    // to the valid rows (a resource of size 0 reads zeros only).  A step lies
    // in one block when the blocks hold a multiple of 32 rows; with 16-row
    // multiples (H16) each 16-row half gets its own resource, in its block.
    // Rows the cache serves: below the split end and below the first new row.
    const int cache_end = min(end, nw);
    auto load = [&](int key0, ExStepData<D, KV8>& st) __attribute__((always_inline)) {
        __amdgpu_buffer_rsrc_t kr[2], vr[2];
        if constexpr (H16) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int row0 = key0 + 16 * x;
                const int valid = min(cache_end - row0, 16);
                int nbytes = 0;
                int64_t off = 0;
                if (valid > 0) {
                    const int blk = block_table[(int64_t)b * max_blocks + row0 / bs];
                    if ((unsigned)blk < (unsigned)num_blocks) {
                        nbytes = (valid - 1) * rs + Ex::ROWB;
                        off = (((int64_t)blk * bs + row0 % bs) * Hkv + g) * Ex::ROWB;
                    }
                }
                kr[x] = make_rsrc(kc + off, nbytes);
                vr[x] = make_rsrc(vc + off, nbytes);
            }
        } else {
            const uint8_t *kp, *vp;
            const int valid = min(cache_end - key0, kDecodeStep);
            int nbytes = valid > 0 ? (valid - 1) * rs + Ex::ROWB : 0;
            if (block_table) {
                const int blk = block_table[(int64_t)b * max_blocks + key0 / bs];
                if ((unsigned)blk >= (unsigned)num_blocks) nbytes = 0;
                const int64_t off = nbytes ? (((int64_t)blk * bs + key0 % bs) * Hkv + g) * Ex::ROWB : 0;
                kp = kc + off;
                vp = vc + off;
            } else {
                kp = kseq + (int64_t)key0 * rs;
                vp = vseq + (int64_t)key0 * rs;
            }
            kr[0] = kr[1] = make_rsrc(kp, nbytes);
            vr[0] = vr[1] = make_rsrc(vp, nbytes);
        }
        ex_load_step<D, KV8, H16>(st, kr, vr, rs, lane);
        if (key0 + kDecodeStep > nw) ex_merge_new_rows<D, KV8>(st, kn, vn, key0, nw, end, T, rs, lane);
    };
    constexpr int stride = NWV * kDecodeStep;
    if constexpr (KV8) {
        // An FP8 step moves half the bytes of a bf16 one: keep the next
        // step's loads in flight while the current step is computed, so a
        // wave has as many bytes outstanding as in the bf16 kernel.
        ExStepData<D, KV8> cur;
        int key0 = kbeg + wave * kDecodeStep;
        if (key0 < end) load(key0, cur);
        for (; key0 < end; key0 += stride) {
            ExStepData<D, KV8> nxt;
            if (key0 + stride < end) load(key0 + stride, nxt);
            ex_stage_k<D, KV>(cur, kt, lane);
            ex_compute_step<D, NT, KV>(cur, kt, key0, end, lane, cs, lo, hi, qB, O, m_run, l_run);
            cur = nxt;
        }
    } else {
        for (int key0 = kbeg + wave * kDecodeStep; key0 < end; key0 += stride) {
            ExStepData<D, KV8> st;
            load(key0, st);
            ex_stage_k<D, KV>(st, kt, lane);
            ex_compute_step<D, NT, KV>(st, kt, key0, end, lane, cs, lo, hi, qB, O, m_run, l_run);
        }
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        l_run[nt] += __shfl_xor(l_run[nt], 16);
        l_run[nt] += __shfl_xor(l_run[nt], 32);
    }
    const float vsc = KV8 ? v_scale[g] : 1.f;
    // Combine the waves' partial results, one 16-row tile at a time: each
    // wave's part of the tile (16 rows x D floats) is staged in its own K
    // tile, which it no longer reads, and after a barrier every thread
    // combines one (row, 8 head-dim values) piece over the waves.
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
        const int items = min(16, R - 16 * nt) * C8;
        for (int it = threadIdx.x; it < items; it += 64 * NWV) {
            const int i = it / C8;
            const int c = (it % C8) * 8;
            const int h = 16 * nt + i;
            const int t = h / gsize, hh = h % gsize;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < NWV; ++w) M = fmaxf(M, sm_m[w * 16 + i]);
            float L = 0.f;
            f32x4 o0 = f32x4{0.f, 0.f, 0.f, 0.f}, o1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NWV; ++w) {
                const float f = M == kNegInf ? 0.f : fast_exp2(sm_m[w * 16 + i] - M);
                L += f * sm_l[w * 16 + i];
                const float* src = reinterpret_cast<const float*>(k_tiles[w]) + i * D + c;
                o0 += f * *reinterpret_cast<const f32x4*>(src);
                o1 += f * *reinterpret_cast<const f32x4*>(src + 4);
            }
            const int64_t row = ((int64_t)b * T + t) * Hq + h0 + hh;
            if (S == 1) {
                const float f = L > 0.f ? vsc / L : 0.f;
                u32x4 o;
                o[0] = pack_bf16x2_rne(o0[0] * f, o0[1] * f);
                o[1] = pack_bf16x2_rne(o0[2] * f, o0[3] * f);
                o[2] = pack_bf16x2_rne(o1[0] * f, o1[1] * f);
                o[3] = pack_bf16x2_rne(o1[2] * f, o1[3] * f);
                *reinterpret_cast<u32x4*>(out + row * D + c) = o;
            } else {
                float* dst = ws_acc + (row * S + s) * D + c;
                *reinterpret_cast<f32x4*>(dst) = o0 * vsc;
                *reinterpret_cast<f32x4*>(dst + 4) = o1 * vsc;
                if (c == 0) {
                    ws_ml[(row * S + s) * 2] = M;
                    ws_ml[(row * S + s) * 2 + 1] = L;
                }
            }
        }
    }
}

// Merge of the split partials of one (b, t, h) row over the splits some
// token of sequence b can see: s in [first / chunk, ceil(n / chunk)).
template <int D>
__global__ __launch_bounds__(64) void decode_ex_merge(const float* __restrict__ ws_acc,
                                                      const float* __restrict__ ws_ml,
                                                      const int32_t* __restrict__ seqlens, int T,
                                                      int Hq, int Lmax, int S, int chunk, int window,
                                                      uint16_t* __restrict__ out) {
    constexpr int PER = D / 64;
    const int64_t row = blockIdx.x;
    const int n = valid_rows(seqlens[row / ((int64_t)T * Hq)], Lmax);
    float acc[PER];
    const float L = merge_split_row<D>(ws_acc, ws_ml, n, row, S, [&](int len, int& s0, int& se) {
        s0 = ex_first_key(len, T, window) / chunk;
        se = min(S, (len + chunk - 1) / chunk);
    }, acc);
    const int c0 = threadIdx.x * PER;
    uint16_t* dst = out + row * D + c0;
    if (PER == 2)
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2_rne(L > 0.f ? acc[0] / L : 0.f, L > 0.f ? acc[PER - 1] / L : 0.f);
    else
        dst[0] = (uint16_t)f32_to_bf16_rne(L > 0.f ? acc[0] / L : 0.f);
}

}  // namespace gqa
