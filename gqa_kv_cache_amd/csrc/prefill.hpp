// Causal GQA prefill on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The prompt attends to itself under a causal mask, so this path is a dense
// contraction and compute-bound ("GQA 深入理解", zulogic.cn, section 5:
// prefill is large matrix multiplication; ttlab lesson, section
// "什么减少，什么不减少": the attention multiplications carry no group term).
//
// A workgroup owns a block of query rows for `hw` query heads of one group;
// its waves share every K and V tile staged in LDS.  Tiles are
// double-buffered: the next tile streams from memory straight into LDS
// (buffer loads with an LDS destination, no registers involved) while the
// current one is consumed.  Each wave keeps 16*MT query rows of one head as
// matrix-core operands in registers and walks the key tiles up to the
// diagonal with an online softmax (reference maximum m, unnormalised O, sum
// of weights).  Scores are formed as S^T = K Q^T so that the result lands
// directly in the A-operand layout of the P*V product, as in the decode
// kernel.  V stays in its natural [key][head dim] layout and is read with
// the gfx950 LDS transpose read, which hands each lane 4 consecutive keys of
// one head-dim value: two such reads form the lane's P*V operand.  P is
// rounded to bf16 for the P*V product; accumulation is fp32.
//
// Softmax reference maximum: the running maximum only moves when a score
// exceeds it by more than 2^8 (in base-2 units); otherwise the weights are
// formed against the old maximum and may reach 256, which fp32 sums and bf16
// weights represent without loss of relative precision.  The sum of weights
// is one more matrix-core product (P times a column of ones), so numerator
// and denominator use the same rounded weights, and the final division makes
// the result independent of the reference.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace gqa {

constexpr int kPrefillWaves = 8;                   // waves per workgroup (2 per SIMD)
constexpr int kPrefillBN = 64;                     // keys per LDS tile
constexpr int kPrefillMT = 2;                      // 16-row query tiles per wave
constexpr int kPrefillRows = 16 * kPrefillMT * 2;  // fewest query rows per workgroup
constexpr float kRescaleSlack = 8.0f;              // log2 of the largest weight allowed
// Reference of a row that has seen no visible key: the lowest finite float.
// Masked (-inf) scores against it give weight 2^-inf = 0 (never NaN), any
// finite score raises it before weights are formed, and a rescale against it
// gives factor 0 (or 1 while the row still has seen nothing).
constexpr float kNoScoreYet = -3.4028234663852886e38f;

template <int D, int NW, int BN> struct PrefillShape {
    static constexpr int KI = D / 32;          // 32-wide head-dim slices of the score MFMA
    static constexpr int NB = D / 16;          // 16-wide head-dim blocks of O
    static constexpr int CPR = D / 8;          // 16-byte chunks per K or V row
    static constexpr int BLK = BN * CPR / 64;  // 1 KB blocks per tile (one direct load each)
    static constexpr int BPW = BLK / NW;       // blocks per wave per tile
    static_assert(BLK % NW == 0, "tile blocks split evenly over waves");
};

// Position of 16-byte chunk c in K tile row r.  The 16 rows one operand
// load reads per pass differ in bits {0,1,3,4} of r; the XOR spreads them
// over all 64 banks: with 256-byte rows (16 chunks) those four bits pick the
// chunk, with 128-byte rows bit 0 already picks the half of the banks and
// bits {1,3,4} pick the chunk.  Bit 2 and bits above 4 are ignored, so rows
// r + 4 and r + 32 share the pattern of row r.
__device__ __forceinline__ int k_pos(int r, int c, int cpr) {
    return cpr == 16 ? c ^ (((r >> 1) & 0xC) | (r & 3)) : c ^ (((r >> 2) & 6) | ((r >> 1) & 1));
}
// Position of chunk c in V tile row r.  One transpose read serves 32 lanes
// per pass: rows 8g + 0..3 and 8g + 8..11.  The XOR with 2(r & 3) spreads
// the four rows of one lane group over distinct banks; bit 3 of the row then
// moves the second group onto the other half of the banks (an offset of 128
// bytes in a 256-byte row, of 32 bytes in a 128-byte row).
__device__ __forceinline__ int v_pos(int r, int c, int cpr) {
    return c ^ ((2 * (r & 3)) % cpr) ^ (((r >> 3) & 1) * (cpr == 16 ? 8 : 2));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D, int MT, int NW, int BN>
__global__ __launch_bounds__(64 * NW) void prefill_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int P, int Hq, int Hkv, int gsize, int hw, int nbgh, int nrb, int causal, int window, float c_log2,
    uint16_t* __restrict__ out) {
    typedef PrefillShape<D, NW, BN> Sh;
    constexpr int KI = Sh::KI;
    constexpr int NB = Sh::NB;
    constexpr int CPR = Sh::CPR;
    constexpr int WR = 16 * MT;
    constexpr int CPT = BN / 32;  // 32-key chunks per tile
    // One array per stage and operand: distinct objects let the compiler
    // see that reads of one stage never wait for direct loads into the other.
    __shared__ u32x4 k_lds0[BN * CPR];
    __shared__ u32x4 k_lds1[BN * CPR];
    __shared__ u32x4 v_lds0[BN * CPR];
    __shared__ u32x4 v_lds1[BN * CPR];
    // Stages are compile-time constants (std::integral_constant).
    auto k_stage = [&](auto st) __attribute__((always_inline)) -> u32x4* {
        if constexpr (decltype(st)::value == 0) return k_lds0;
        else return k_lds1;
    };
    auto v_stage = [&](auto st) __attribute__((always_inline)) -> u32x4* {
        if constexpr (decltype(st)::value == 0) return v_lds0;
        else return v_lds1;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar: everything derived from it is wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // rows at or past P read as zero
    const int valid_bytes = (P - 1) * ks2 + D * 2;
    __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), (short)0, valid_bytes, 0x00020000);
    __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), (short)0, valid_bytes, 0x00020000);

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

    // K operand slots.  Row 4 + r of a chunk swizzles like row r (the XOR
    // ignores bit 2), so sub-tile t = 1 is sub-tile 0 shifted by 4 rows.
    int ka_slot[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int r = 8 * (col >> 2) + (col & 3);
        ka_slot[i] = r * CPR + k_pos(r, 4 * i + grp, CPR);
    }
    // V transpose reads: lane (L = lane % 16, grp) names row 8grp + L/4 and
    // the 8 bytes of head-dims 16e + 4(L%4) .. +3; it receives keys
    // 8grp + 0..3 (+4 for the second read) of head-dim 16e + L.
    int vt_byte[NB];
    {
        const int L = lane & 15, m = L & 3;
        const int r = 8 * grp + (L >> 2);
#pragma unroll
        for (int e = 0; e < NB; ++e)
            vt_byte[e] = r * CPR * 16 + v_pos(r, 2 * e + (m >> 1), CPR) * 16 + 8 * (m & 1);
    }
    // Tile fill: wave w streams 1 KB blocks w, w + NW, ... straight into
    // LDS; lane l of a block lands in slot 64*block + l, so it fetches the
    // global chunk that the swizzle places there (both swizzles are XORs, so
    // position and chunk map onto each other the same way).
    int k_off[Sh::BPW], v_off[Sh::BPW];
#pragma unroll
    for (int x = 0; x < Sh::BPW; ++x) {
        const int slot = 64 * (wave + NW * x) + lane;
        const int r = slot / CPR, pos = slot % CPR;
        k_off[x] = r * ks2 + 16 * k_pos(r, pos, CPR);
        v_off[x] = r * ks2 + 16 * v_pos(r, pos, CPR);
    }
    // The whole byte offset goes in the per-lane operand, so the range check
    // of the buffer resource zero-fills every row at or past P.
    auto fill = [&](auto stage, int j0) __attribute__((always_inline)) {
        u32x4* kl = k_stage(stage);
        u32x4* vl = v_stage(stage);
        const int base = j0 * ks2;
#pragma unroll
        for (int x = 0; x < Sh::BPW; ++x) {
            const int blk = wave + NW * x;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)&kl[64 * blk], 16u,
                                                     (unsigned)(base + k_off[x]), 0u, 0u, 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)&vl[64 * blk], 16u,
                                                     (unsigned)(base + v_off[x]), 0u, 0u, 0u);
        }
    };

    // O accumulators (lane: head-dims 16e + col of rows 16mt + 4grp + r);
    // osum accumulates P times a column of ones: the sum of the bf16 weights
    // actually used, per row in the same layout.
    f32x4 O[MT][NB];
    f32x4 osum[MT];
    float m_ref[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_ref[mt] = kNoScoreYet;
        osum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < NB; ++e) O[mt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // S^T = K Q^T of chunk c of the staged tile for every row tile; each K
    // fragment serves all MT tiles.
    auto scores = [&](auto stage, int c, f32x4 (&sc)[MT][2]) __attribute__((always_inline)) {
        const u32x4* kl = k_stage(stage);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sc[mt][0] = sc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const u32x4 kA = kl[ka_slot[i] + (32 * c + 4 * t) * CPR];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    sc[mt][t] = mfma16x16x32(as_bf16x8(kA), qB[mt][i], sc[mt][t]);
            }
    };
    // Causal / tail mask of the chunk starting at key kc0.
    auto mask = [&](int kc0, f32x4 (&sc)[MT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int qrow = iw + 16 * mt + col;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kc0 + 8 * grp + 4 * t + r;
                    if (key >= P || (causal && key > qrow) || (window > 0 && key <= qrow - window))
                        sc[mt][t][r] = kNegInf;
                }
        }
    };
    // Move the reference maxima only when a weight would exceed 2^slack.
    // IEEE maximum (NaN-propagating) needs no canonicalisation of the
    // matrix-core results, so 8 scores take 4 three-input instructions.
    auto update_max = [&](const f32x4 (&sc)[MT][2]) __attribute__((always_inline)) {
        float mx[MT];
        bool grow = false;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[mt][0][0], sc[mt][0][1]), sc[mt][0][2]);
            const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[mt][0][3], sc[mt][1][0]), sc[mt][1][1]);
            const float c = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[mt][1][2], sc[mt][1][3]), a);
            mx[mt] = __builtin_elementwise_maximum(b, c);
            grow |= mx[mt] * cs > m_ref[mt] + kRescaleSlack;
        }
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
                    for (int e = 0; e < NB; ++e) O[mt][e][r] *= ar;
                }
            }
        }
    };
    // Weights 2^(s*|c| - m) rounded to bf16, as the A operand of P*V.
    auto weights = [&](const f32x4 (&sc)[MT][2], u32x4 (&pa)[MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float mr = m_ref[mt];
            float w[8];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) w[4 * t + r] = fast_exp2(__builtin_fmaf(sc[mt][t][r], cs, -mr));
#pragma unroll
            for (int j = 0; j < 4; ++j) pa[mt][j] = pack_bf16x2_rne(w[2 * j], w[2 * j + 1]);
        }
    };
    // O += P V and the weight sums; each V fragment serves all MT tiles.
    auto accumulate = [&](auto stage, int c, const u32x4 (&pa)[MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) osum[mt] = mfma16x16x32(as_bf16x8(pa[mt]), ones, osum[mt]);
        const char* vbase = reinterpret_cast<const char*>(v_stage(stage) + 32 * c * CPR);
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + vt_byte[e]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + vt_byte[e] + 4 * CPR * 16));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 vF = u32x4{l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                O[mt][e] = mfma16x16x32(as_bf16x8(pa[mt]), as_bf16x8(vF), O[mt][e]);
        }
    };

    const int kv_end = causal ? min(P, i0 + rows_wg) : P;
    const int wave_last_row = min(iw + WR, P) - 1;
    const int ntiles = (kv_end + BN - 1) / BN;
    // sliding window (causal only): row i sees keys [i - window + 1, i]; the
    // workgroup starts at the first tile its first row can see
    const int jt_lo = window > 0 ? max(0, i0 - window + 1) / BN : 0;
    // keys this wave needs: up to kv_end, and up to its last row when causal
    const int lim = causal ? min(kv_end, wave_last_row + 1) : kv_end;

    typedef std::integral_constant<int, 0> Stage0;
    typedef std::integral_constant<int, 1> Stage1;
    // One key tile: prefetch the next tile into the other stage (released by
    // every wave at the previous barrier), consume this one, then wait for
    // this wave's direct loads and meet the other waves.
    auto tile = [&](auto stage, int jt) __attribute__((always_inline)) {
        typedef std::integral_constant<int, 1 - decltype(stage)::value> Other;
        const int j0 = jt * BN;
        if (jt + 1 < ntiles) fill(Other{}, j0 + BN);
        const bool full = j0 + BN <= lim && j0 + BN <= P && (!causal || j0 + BN - 1 <= iw) &&
                          (window <= 0 || j0 > wave_last_row - window);
        if (full) {
#pragma unroll 1
            for (int c = 0; c < CPT; ++c) {
                f32x4 sc[MT][2];
                scores(stage, c, sc);
                update_max(sc);
                u32x4 pa[MT];
                weights(sc, pa);
                accumulate(stage, c, pa);
            }
        } else {
            // Diagonal or tail tile: masked chunks, up to the wave's last key.
#pragma unroll 1
            for (int c = 0; c < CPT; ++c) {
                const int kc0 = j0 + 32 * c;
                if (kc0 >= lim) break;
                if (window > 0 && kc0 + 31 <= iw - window) continue;  // below every row's window
                f32x4 sc[MT][2];
                scores(stage, c, sc);
                mask(kc0, sc);
                update_max(sc);
                u32x4 pa[MT];
                weights(sc, pa);
                accumulate(stage, c, pa);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
        __syncthreads();
    };

    fill(Stage0{}, jt_lo * BN);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int jt = jt_lo; jt < ntiles; jt += 2) {
        tile(Stage0{}, jt);
        if (jt + 1 < ntiles) tile(Stage1{}, jt + 1);
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = iw + 16 * mt + 4 * grp + r;
            const float l = osum[mt][r];
            if (row < P) {
                // lane holds head-dims 16e + col of the row
                uint16_t* dst = out + ((int64_t)b * P + row) * qs + (int64_t)head * D + col;
                const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
                for (int e = 0; e < NB; ++e) dst[16 * e] = (uint16_t)f32_to_bf16_rne(O[mt][e][r] * inv);
            }
        }
    }
}

// Host-side launch; returns false if the launch itself failed.
template <int D, int MT, int NW, int BN>
inline bool launch_prefill_cfg(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int P,
                               int Hq, int Hkv, bool causal, int window, float c_log2, uint16_t* out,
                               hipStream_t stream) {
    const int gsize = Hq / Hkv;
    const int hw = gsize % 4 == 0 ? 4 : gsize % 2 == 0 ? 2 : 1;
    const int rows_wg = 16 * MT * (NW / hw);
    const int nrb = (P + rows_wg - 1) / rows_wg;
    const int nbgh = B * Hkv * (gsize / hw);
    dim3 grid((unsigned)((int64_t)nbgh * nrb));
    dim3 block(64 * NW);
    hipLaunchKernelGGL((prefill_bf16<D, MT, NW, BN>), grid, block, 0, stream, q, k, v, P, Hq,
                       Hkv, gsize, hw, nbgh, nrb, causal ? 1 : 0, window, c_log2, out);
    return hipGetLastError() == hipSuccess;
}

inline bool launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int P,
                           int Hq, int Hkv, int d, bool causal, int window, float c_log2,
                           uint16_t* out, hipStream_t stream) {
    if (d == 128)
        return launch_prefill_cfg<128, kPrefillMT, kPrefillWaves, kPrefillBN>(q, k, v, B, P, Hq, Hkv, causal, window, c_log2, out, stream);
    return launch_prefill_cfg<64, kPrefillMT, kPrefillWaves, kPrefillBN>(q, k, v, B, P, Hq, Hkv, causal, window, c_log2, out, stream);
}

}  // namespace gqa
