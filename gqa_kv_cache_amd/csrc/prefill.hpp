// Causal GQA prefill on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The prompt attends to itself under a causal mask, so this path is a dense
// contraction and compute-bound ("GQA 深入理解", zulogic.cn, section 5:
// prefill is large matrix multiplication; ttlab lesson, section
// "什么减少，什么不减少": the attention multiplications carry no group term).
//
// A workgroup owns a block of query rows for `hw` query heads of one group;
// its four waves share every K and V tile staged in LDS.  Each wave keeps
// 16*MT query rows of one head in registers and walks the key tiles up to
// the diagonal with an online softmax (running max m, sum l, unnormalised
// O).  Scores are formed as S^T = K Q^T so that the result lands directly in
// the A-operand layout of the P*V product, as in the decode kernel.  V is
// staged transposed ([head dim][key]) so each lane's P*V operand is 8
// consecutive keys of one head-dim value.  P is rounded to bf16 for the
// P*V product; accumulation is fp32.
#pragma once

#include "common.hpp"

namespace gqa {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillBN = 64;  // keys per LDS tile
constexpr int kPrefillMT = 2;   // 16-row query tiles per wave
constexpr int kPrefillRows = 16 * kPrefillMT;  // fewest query rows per workgroup

template <int D, int MT>
__global__ __launch_bounds__(kPrefillThreads) void prefill_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int P, int Hq, int Hkv, int gsize, int hw, int nbgh, int nrb, int causal, float c_log2,
    uint16_t* __restrict__ out) {
    constexpr int KI = D / 32;
    constexpr int EPL = D / 16;
    constexpr int WR = 16 * MT;
    constexpr int BN = kPrefillBN;
    constexpr int KS = D + 8;   // K tile row stride (elements), padded
    constexpr int VS = BN + 8;  // V^T tile row stride (elements), padded
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    // (b, g, head subset) varies fastest; the latest (heaviest) row blocks go first.
    const int bgh = blockIdx.x % nbgh;
    const int rb = nrb - 1 - blockIdx.x / nbgh;
    const int hsets = gsize / hw;
    const int hs = bgh % hsets;
    const int bg = bgh / hsets;
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int rows_wg = WR * (4 / hw);
    const int i0 = rb * rows_wg;
    const int head = g * gsize + hs * hw + (wave % hw);
    const int iw = i0 + (wave / hw) * WR;

    const int64_t qs = (int64_t)Hq * D;
    const int64_t ks = (int64_t)Hkv * D;
    const uint16_t* qb = q + (int64_t)b * P * qs + (int64_t)head * D;
    const uint16_t* kb = k + (int64_t)b * P * ks + (int64_t)g * D;
    const uint16_t* vb = v + (int64_t)b * P * ks + (int64_t)g * D;

    bf16x8 qB[MT][KI];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = iw + 16 * mt + col;
        const bool ok = row < P;
        const uint16_t* qp = qb + (int64_t)(ok ? row : 0) * qs + 8 * grp;
#pragma unroll
        for (int i = 0; i < KI; ++i) qB[mt][i] = as_bf16x8(load16(qp + 32 * i, ok));
    }

    f32x4 O[MT][EPL];
    float m_run[MT], l_run[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = kNegInf;
        l_run[mt] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) O[mt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int kv_end = causal ? min(P, i0 + rows_wg) : P;
    const int wave_last_row = min(iw + WR, P) - 1;

    for (int j0 = 0; j0 < kv_end; j0 += BN) {
        __syncthreads();
        // K tile, natural layout: 16-byte pieces, 8 head-dim values each.
        for (int idx = threadIdx.x; idx < BN * (D / 8); idx += kPrefillThreads) {
            const int r = idx / (D / 8);
            const int cp = (idx % (D / 8)) * 8;
            const int key = j0 + r;
            *reinterpret_cast<u32x4*>(k_lds + r * KS + cp) =
                load16(kb + (int64_t)(key < P ? key : 0) * ks + cp, key < P);
        }
        // V tile, transposed: each thread moves 4 keys x 8 head-dim values.
        for (int idx = threadIdx.x; idx < (BN / 4) * (D / 8); idx += kPrefillThreads) {
            const int db = idx % (D / 8);
            const int k4 = idx / (D / 8);
            u32x4 w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = j0 + 4 * k4 + r;
                w[r] = load16(vb + (int64_t)(key < P ? key : 0) * ks + 8 * db, key < P);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int x = e >> 1;
                const uint32_t lo = (e & 1) ? pack_hi16(w[0][x], w[1][x]) : pack_lo16(w[0][x], w[1][x]);
                const uint32_t hi = (e & 1) ? pack_hi16(w[2][x], w[3][x]) : pack_lo16(w[2][x], w[3][x]);
                *reinterpret_cast<u32x2*>(vt_lds + (8 * db + e) * VS + 4 * k4) = u32x2{lo, hi};
            }
        }
        __syncthreads();

#pragma unroll
        for (int c = 0; c < BN / 32; ++c) {
            const int kc0 = j0 + 32 * c;
            if (kc0 >= kv_end) break;
            if (causal && kc0 > wave_last_row) continue;
            // A operand of S^T = K Q^T: row `col` of sub-tile t is key 8*(col/4) + 4t + col%4.
            u32x4 kA[2][KI];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rt = 32 * c + 8 * (col >> 2) + 4 * t + (col & 3);
#pragma unroll
                for (int i = 0; i < KI; ++i)
                    kA[t][i] = *reinterpret_cast<const u32x4*>(k_lds + rt * KS + 32 * i + 8 * grp);
            }
            // B operand of O += P V: head-dim value EPL*col + e, keys 8*grp .. 8*grp+7.
            u32x4 vF[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                vF[e] = *reinterpret_cast<const u32x4*>(vt_lds + (EPL * col + e) * VS + 32 * c + 8 * grp);

#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int qrow = iw + 16 * mt + col;
                float p[8];
                float mx = kNegInf;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < KI; ++i) acc = mfma16x16x32(as_bf16x8(kA[t][i]), qB[mt][i], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kc0 + 8 * grp + 4 * t + r;
                        const bool ok = key < P && (!causal || key <= qrow);
                        const float sv = ok ? acc[r] * c_log2 : kNegInf;
                        p[4 * t + r] = sv;
                        mx = fmaxf(mx, sv);
                    }
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[mt], mx);
                const float alpha = fast_exp2(m_run[mt] - m_new);
                m_run[mt] = m_new;
                float psum = 0.f;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    p[x] = fast_exp2(p[x] - m_new);
                    psum += p[x];
                }
                l_run[mt] = l_run[mt] * alpha + psum;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) O[mt][e][r] *= ar;
                }
                u32x4 pa;
#pragma unroll
                for (int j = 0; j < 4; ++j) pa[j] = pack_bf16x2_rne(p[2 * j], p[2 * j + 1]);
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    O[mt][e] = mfma16x16x32(as_bf16x8(pa), as_bf16x8(vF[e]), O[mt][e]);
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        l_run[mt] += __shfl_xor(l_run[mt], 16);
        l_run[mt] += __shfl_xor(l_run[mt], 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = iw + 16 * mt + 4 * grp + r;
            const float l = __shfl(l_run[mt], 4 * grp + r);
            if (row < P) {
                uint16_t* dst = out + ((int64_t)b * P + row) * qs + (int64_t)head * D + EPL * col;
                const float inv = l > 0.f ? 1.f / l : 0.f;
                if constexpr (EPL == 8) {
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2_rne(O[mt][2 * j][r] * inv, O[mt][2 * j + 1][r] * inv);
                    *reinterpret_cast<u32x4*>(dst) = o;
                } else {
                    u32x2 o;
#pragma unroll
                    for (int j = 0; j < 2; ++j) o[j] = pack_bf16x2_rne(O[mt][2 * j][r] * inv, O[mt][2 * j + 1][r] * inv);
                    *reinterpret_cast<u32x2*>(dst) = o;
                }
            }
        }
    }
}

// Host-side launch; returns false if the launch itself failed.
inline bool launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int P,
                           int Hq, int Hkv, int d, bool causal, float c_log2, uint16_t* out,
                           hipStream_t stream) {
    const int gsize = Hq / Hkv;
    const int hw = gsize % 4 == 0 ? 4 : gsize % 2 == 0 ? 2 : 1;
    const int rows_wg = kPrefillRows * (4 / hw);
    const int nrb = (P + rows_wg - 1) / rows_wg;
    const int nbgh = B * Hkv * (gsize / hw);
    dim3 grid((unsigned)((int64_t)nbgh * nrb));
    dim3 block(kPrefillThreads);
    if (d == 128)
        hipLaunchKernelGGL((prefill_bf16<128, kPrefillMT>), grid, block, 0, stream, q, k, v, P, Hq, Hkv,
                           gsize, hw, nbgh, nrb, causal ? 1 : 0, c_log2, out);
    else
        hipLaunchKernelGGL((prefill_bf16<64, kPrefillMT>), grid, block, 0, stream, q, k, v, P, Hq, Hkv,
                           gsize, hw, nbgh, nrb, causal ? 1 : 0, c_log2, out);
    return hipGetLastError() == hipSuccess;
}

}  // namespace gqa
