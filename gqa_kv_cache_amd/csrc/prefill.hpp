// Causal GQA prefill on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The prompt attends to itself under a causal mask, so this path is a dense
// contraction and compute-bound ("GQA 深入理解", zulogic.cn, section 5:
// prefill is large matrix multiplication; ttlab lesson, section
// "什么减少，什么不减少": the attention multiplications carry no group term).
//
// A workgroup owns a block of query rows for `hw` query heads of one group;
// its four waves share every K and V tile staged in LDS (double-buffered:
// the next tile is loaded into registers while the current one is consumed).
// Each wave keeps 16*MT query rows of one head in registers and walks the
// key tiles up to the diagonal with an online softmax (running max m, sum l,
// unnormalised O).  Scores are formed as S^T = K Q^T so that the result
// lands directly in the A-operand layout of the P*V product, as in the
// decode kernel.  V is staged transposed ([head dim][key]) so each lane's
// P*V operand is 8 consecutive keys of one head-dim value.  P is rounded to
// bf16 for the P*V product; accumulation is fp32.
//
// Softmax reference maximum: the running maximum only moves when a score
// exceeds it by more than 2^8 (in base-2 units); otherwise the weights are
// formed against the old maximum and may reach 256, which fp32 sums and bf16
// weights represent without loss of relative precision.  The final division
// by the sum of weights makes the result independent of the reference.
#pragma once

#include "common.hpp"

namespace gqa {

constexpr int kPrefillWaves = 8;                    // waves per workgroup (2 per SIMD)
constexpr int kPrefillBN = 64;                      // keys per LDS tile
constexpr int kPrefillMT = 2;                       // 16-row query tiles per wave
constexpr int kPrefillRows = 16 * kPrefillMT * 2;   // fewest query rows per workgroup
constexpr float kRescaleSlack = 8.0f;          // log2 of the largest weight allowed

template <int D, int NW, int BN> struct PrefillShape {
    static constexpr int NTH = 64 * NW;  // threads per workgroup
    static constexpr int KI = D / 32;    // 32-wide head-dim slices of the score MFMA
    static constexpr int EPL = D / 16;   // head-dim values per lane in O
    static constexpr int CPR = D / 8;    // 16-byte chunks per K row
    static constexpr int KCH = BN * CPR / NTH;                  // K chunks per thread per tile
    static_assert(BN * CPR % NTH == 0, "K tile splits evenly over threads");
    static constexpr int VITEMS = (BN / 4) * (D / 8);           // V 4x8 blocks per tile
    static constexpr int VCH = (VITEMS + NTH - 1) / NTH;        // per thread
};

// Position of 16-byte chunk c of K tile row r: rows read together by one
// MFMA operand load differ in bits {0,1,3,4} of r, which select the XOR.
__device__ __forceinline__ int k_slot(int r, int c, int cpr) {
    return r * cpr + (c ^ ((((r >> 1) & 0xC) | (r & 3)) % cpr));
}
// V^T tile: each head-dim value d holds BN keys as BN/8 chunks of 8 keys;
// DPL = 16/(BN/8) consecutive values share one 256-byte line of 16 chunks.
// The XOR spreads the 16 values one MFMA operand load reads (d = 8*lane + e)
// over distinct chunk positions.
template <int BN>
__device__ __forceinline__ int v_slot(int d, int kc) {
    static_assert(BN == 32 || BN == 64 || BN == 128, "key tile of 32, 64 or 128");
    constexpr int CPD = BN / 8;
    constexpr int DPL = 16 / CPD;
    constexpr int SH = DPL == 1 ? 3 : DPL == 2 ? 2 : 1;  // (line >> SH) == d / 8
    const int line = d / DPL;
    return line * 16 + ((CPD * (d % DPL) + kc) ^ ((line >> SH) & 15));
}

template <int D, int MT, int NW, int BN, bool UNROLL>
__global__ __launch_bounds__(64 * NW) void prefill_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int P, int Hq, int Hkv, int gsize, int hw, int nbgh, int nrb, int causal, float c_log2,
    uint16_t* __restrict__ out) {
    typedef PrefillShape<D, NW, BN> Sh;
    constexpr int KI = Sh::KI;
    constexpr int EPL = Sh::EPL;
    constexpr int CPR = Sh::CPR;
    constexpr int WR = 16 * MT;
    constexpr int NTH = Sh::NTH;
    __shared__ u32x4 k_lds[2][BN * CPR];
    __shared__ u32x4 v_lds[2][D * BN / 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const int rows_wg = WR * (NW / hw);
    const int i0 = rb * rows_wg;
    const int head = g * gsize + hs * hw + (wave % hw);
    const int iw = i0 + (wave / hw) * WR;

    const int64_t qs = (int64_t)Hq * D;
    const int ks2 = Hkv * D * 2;  // bytes between consecutive positions of one KV head
    const uint16_t* qb = q + (int64_t)b * P * qs + (int64_t)head * D;
    const uint16_t* kb = k + (int64_t)b * P * Hkv * D + (int64_t)g * D;
    const uint16_t* vb = v + (int64_t)b * P * Hkv * D + (int64_t)g * D;
    const int valid_bytes = (P - 1) * ks2 + D * 2;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), (short)0, valid_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), (short)0, valid_bytes, 0x00020000);

    // Query rows of this wave as B operands (lane: row iw + 16mt + col).
    bf16x8 qB[MT][KI];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = iw + 16 * mt + col;
        const bool ok = row < P;
        const uint16_t* qp = qb + (int64_t)(ok ? row : 0) * qs + 8 * grp;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            u32x4 w = load16(qp + 32 * i, ok);
            // A negative scale is applied as a positive one to -q (exact in bf16).
            if (c_log2 < 0.f) w ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            qB[mt][i] = as_bf16x8(w);
        }
    }
    // |scale| * log2(e), kept away from zero so masked (-inf) scores still
    // give zero weight; a zero scale then yields equal weights as it should.
    const float cs = fmaxf(fabsf(c_log2), 1e-30f);
    const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    // Lane-constant LDS slots of the operand reads.
    int ka_slot[2][KI];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < KI; ++i) ka_slot[t][i] = k_slot(8 * (col >> 2) + 4 * t + (col & 3), 4 * i + grp, CPR);
    // Chunk kc = 4c + grp of V^T: bit 2 of the unswizzled slot is c (64-key
    // tiles), so the slot for chunk c is the c = 0 slot with bit 2 flipped.
    int vb_slot[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) vb_slot[e] = v_slot<BN>(EPL * col + e, grp);

    // Tile fill: K as 16-byte chunks, V as blocks of 4 keys x 8 head-dim values.
    u32x4 kst[Sh::KCH];
    u32x4 vst[Sh::VCH][4];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int x = 0; x < Sh::KCH; ++x) {
            const int idx = tid + NTH * x;
            const int r = idx / CPR, cp = idx % CPR;
            kst[x] = __builtin_amdgcn_raw_buffer_load_b128(kr, (j0 + r) * ks2 + 16 * cp, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < Sh::VCH; ++x) {
            const int idx = tid + NTH * x;
            if (Sh::VITEMS % NTH != 0 && idx >= Sh::VITEMS) break;
            const int db = idx % (D / 8), k4 = idx / (D / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vst[x][r] = __builtin_amdgcn_raw_buffer_load_b128(vr, (j0 + 4 * k4 + r) * ks2 + 16 * db, 0, 0);
        }
    };
    auto stash = [&](int stage) {
#pragma unroll
        for (int x = 0; x < Sh::KCH; ++x) {
            const int idx = tid + NTH * x;
            k_lds[stage][k_slot(idx / CPR, idx % CPR, CPR)] = kst[x];
        }
#pragma unroll
        for (int x = 0; x < Sh::VCH; ++x) {
            const int idx = tid + NTH * x;
            if (Sh::VITEMS % NTH != 0 && idx >= Sh::VITEMS) break;
            const int db = idx % (D / 8), k4 = idx / (D / 8);
            u32x2* vl = reinterpret_cast<u32x2*>(v_lds[stage]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int xw = e >> 1;
                const uint32_t lo = (e & 1) ? pack_hi16(vst[x][0][xw], vst[x][1][xw]) : pack_lo16(vst[x][0][xw], vst[x][1][xw]);
                const uint32_t hi = (e & 1) ? pack_hi16(vst[x][2][xw], vst[x][3][xw]) : pack_lo16(vst[x][2][xw], vst[x][3][xw]);
                // keys 4*k4 .. 4*k4+3 are the (k4 & 1) half of chunk k4 >> 1
                vl[2 * v_slot<BN>(8 * db + e, k4 >> 1) + (k4 & 1)] = u32x2{lo, hi};
            }
        }
    };

    // O accumulators; osum accumulates P times a column of ones, i.e. the sum
    // of the bf16 weights actually used, per row in the O row layout.
    f32x4 O[MT][EPL];
    f32x4 osum[MT];
    float m_ref[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_ref[mt] = kNegInf;
        osum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < EPL; ++e) O[mt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int kv_end = causal ? min(P, i0 + rows_wg) : P;
    const int wave_last_row = min(iw + WR, P) - 1;
    const int ntiles = (kv_end + BN - 1) / BN;

    fetch(0);
    stash(0);
    __syncthreads();
    for (int jt = 0; jt < ntiles; ++jt) {
        const int stage = jt & 1;
        const int j0 = jt * BN;
        if (jt + 1 < ntiles) fetch(j0 + BN);

#pragma unroll
        for (int c = 0; c < BN / 32; ++c) {
            if (!UNROLL) __builtin_amdgcn_sched_barrier(0);
            const int kc0 = j0 + 32 * c;
            if (kc0 >= kv_end) break;
            if (causal && kc0 > wave_last_row) continue;
            // chunk keys reach past P or past this wave's first row: mask
            const bool edge = (kc0 + 31 >= P) || (causal && kc0 + 31 > iw);
            // S^T = K Q^T for every row tile; each K fragment serves all MT tiles.
            f32x4 sacc[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sacc[mt][0] = sacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < KI; ++i) {
                    const u32x4 kA = k_lds[stage][ka_slot[t][i] + 32 * c * CPR];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        sacc[mt][t] = mfma16x16x32(as_bf16x8(kA), qB[mt][i], sacc[mt][t]);
                }
            // raw scores; masked ones become -inf (weight exp2(-inf) = 0)
            float p[MT][8];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[mt][4 * t + r] = sacc[mt][t][r];
            if (edge) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int qrow = iw + 16 * mt + col;
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const int key = kc0 + 8 * grp + x;
                        if (key >= P || (causal && key > qrow)) p[mt][x] = kNegInf;
                    }
                }
            }
            float mx[MT];
            bool grow = false;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                mx[mt] = p[mt][0];
#pragma unroll
                for (int x = 1; x < 8; ++x) mx[mt] = fmaxf(mx[mt], p[mt][x]);
                grow |= mx[mt] * cs > m_ref[mt] + kRescaleSlack;
            }
            // Move the reference maxima only when a weight would exceed 2^slack.
            if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    float rm = fmaxf(mx[mt], __shfl_xor(mx[mt], 16));
                    rm = fmaxf(rm, __shfl_xor(rm, 32));
                    const float m_new = fmaxf(m_ref[mt], rm * cs);
                    const float alpha = fast_exp2(m_ref[mt] - m_new);
                    m_ref[mt] = m_new;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float ar = __shfl(alpha, 4 * grp + r);
                        osum[mt][r] *= ar;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) O[mt][e][r] *= ar;
                    }
                }
            }
            u32x4 pa[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float mr = m_ref[mt];
#pragma unroll
                for (int x = 0; x < 8; ++x) p[mt][x] = fast_exp2(__builtin_fmaf(p[mt][x], cs, -mr));
#pragma unroll
                for (int j = 0; j < 4; ++j) pa[mt][j] = pack_bf16x2_rne(p[mt][2 * j], p[mt][2 * j + 1]);
                osum[mt] = mfma16x16x32(as_bf16x8(pa[mt]), ones, osum[mt]);
            }
            // O += P V; each V fragment serves all MT tiles.
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const u32x4 vF = v_lds[stage][vb_slot[e] ^ (c << 2)];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    O[mt][e] = mfma16x16x32(as_bf16x8(pa[mt]), as_bf16x8(vF), O[mt][e]);
            }
        }
        if (jt + 1 < ntiles) stash(stage ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = iw + 16 * mt + 4 * grp + r;
            const float l = osum[mt][r];
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
template <int D, int MT, int NW, int BN, bool UNROLL>
inline bool launch_prefill_cfg(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int P,
                               int Hq, int Hkv, bool causal, float c_log2, uint16_t* out,
                               hipStream_t stream) {
    const int gsize = Hq / Hkv;
    const int hw = gsize % 4 == 0 ? 4 : gsize % 2 == 0 ? 2 : 1;
    const int rows_wg = 16 * MT * (NW / hw);
    const int nrb = (P + rows_wg - 1) / rows_wg;
    const int nbgh = B * Hkv * (gsize / hw);
    dim3 grid((unsigned)((int64_t)nbgh * nrb));
    dim3 block(64 * NW);
    hipLaunchKernelGGL((prefill_bf16<D, MT, NW, BN, UNROLL>), grid, block, 0, stream, q, k, v, P, Hq,
                       Hkv, gsize, hw, nbgh, nrb, causal ? 1 : 0, c_log2, out);
    return hipGetLastError() == hipSuccess;
}

inline bool launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int P,
                           int Hq, int Hkv, int d, bool causal, float c_log2, uint16_t* out,
                           hipStream_t stream) {
    if (d == 128)
        return launch_prefill_cfg<128, kPrefillMT, kPrefillWaves, kPrefillBN, false>(q, k, v, B, P, Hq, Hkv, causal, c_log2, out, stream);
    return launch_prefill_cfg<64, kPrefillMT, kPrefillWaves, kPrefillBN, false>(q, k, v, B, P, Hq, Hkv, causal, c_log2, out, stream);
}

}  // namespace gqa
