// Causal GQA prefill on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The prompt attends to itself under a causal mask, so this path is a dense
// contraction and compute-bound ("GQA 深入理解", zulogic.cn, section 5:
// prefill is large matrix multiplication; ttlab lesson, section
// "什么减少，什么不减少": the attention multiplications carry no group term).
//
// A workgroup of eight waves owns a block of query rows for `hw` query heads
// of one group; its waves share every K and V chunk staged in LDS (GQA: the
// group shares K/V).  Each wave keeps 16*MT query rows of one head as
// matrix-core operands in registers and walks the 32-key chunks up to the
// diagonal with an online softmax.  Scores are formed as S^T = K Q^T so the
// result lands directly in the A-operand layout of the P*V product.  V stays
// in its natural [key][head dim] layout and is read with the gfx950 LDS
// transpose read.  P is rounded to bf16 for the P*V product; accumulation is
// fp32; the sum of weights is one more matrix-core product (P times a column
// of ones), so numerator and denominator use the same rounded weights.
//
// Software pipeline.  The row tiles of a wave form two halves.  Step n
// finishes chunk n and starts chunk n+1 in two phases, each pairing a block
// of matrix-core products with independent vector work:
//   phase 1: scores S(n+1) = K(n+1) Q^T (all row tiles)  ||  upper-half weights of chunk n
//   phase 2: O += P(n) V(n) and the weight sums          ||  lower-half weights of chunk n+1
// so the matrix cores and the vector ALUs of a SIMD work at the same time
// instead of taking turns.  Source order inside a phase is fixed with
// scheduling barriers, and every formed weight is pinned where it is made.
// Every step runs the same code: the step before a wave's first chunk
// finishes an empty chunk (weights zero, V rows finite), and the step after
// its last chunk starts a chunk the mask removes entirely.
//
// Softmax references.  A row's reference is an integer (base-2 units) that
// only moves when a new score exceeds it by more than 2^8; otherwise weights
// may reach 256, which fp32 sums and bf16 weights hold without loss of
// relative precision, and the final division by the matching sum makes the
// result independent of the reference.  The check runs once per step, a few
// products into phase 2 (the new scores have landed by then); a move scales
// O, the sums and the bf16 weights still feeding this P*V by the same exact
// power of two.
//
// LDS.  K and V of each chunk rotate through four stages (64 KB in all at
// head dim 128, so every LDS address folds into the instructions' 16-bit
// offsets).  Chunks stream from memory straight into LDS (buffer loads with
// an LDS destination).  One barrier per step: at the barrier before step n,
// K(n+4) and V(n+3) start loading over K(n) and V(n-1), whose last reader was
// step n-1.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace gqa {

constexpr int kPrefillWaves = 8;                   // waves per workgroup (2 per SIMD)
constexpr int kPrefillMT = 2;                      // 16-row query tiles per wave
constexpr int kPrefillRows = 16 * kPrefillMT * 2;  // fewest query rows per workgroup
constexpr int kPrefillChunk = 32;                  // keys per pipeline step
constexpr float kRescaleSlack = 8.0f;              // log2 of the largest weight allowed
// Reference of a row that has seen no visible key: the lowest finite float.
// Masked (-inf) scores against it give weight 2^-inf = 0 (never NaN), any
// finite score raises it before weights are formed, and a rescale against it
// gives factor 0 (or 1 while the row still has seen nothing).
constexpr float kNoScoreYet = -3.4028234663852886e38f;

// Position of 16-byte piece c in row r of a staged K chunk.  The 16 rows one
// operand load reads per pass differ in bits {0,1,3,4} of r; the XOR spreads
// them over all 64 banks: with 256-byte rows (16 pieces) those four bits pick
// the piece, with 128-byte rows bit 0 already picks the half of the banks and
// bits {1,3,4} pick the piece.  Bit 2 is ignored, so the operand rows of the
// second 16-key half (r + 4) share the pattern of the first.
__device__ __forceinline__ int k_pos(int r, int c, int cpr) {
    return cpr == 16 ? c ^ (((r >> 1) & 0xC) | (r & 3)) : c ^ (((r >> 2) & 6) | ((r >> 1) & 1));
}
// Position of piece c in row r of a staged V chunk.  One transpose read serves 32 lanes
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

template <int N> using IntC = std::integral_constant<int, N>;

// Slot of weight u among the sl matrix-core slots of a phase that forms nw
// weights per lane (spread evenly).
__host__ __device__ constexpr int wslot(int u, int sl, int nw) { return u * sl / nw; }

template <int D, int MT, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int P, int Hq, int Hkv, int gsize, int hw, int nbgh, int nrb, int causal, int window, float c_log2,
    uint16_t* __restrict__ out) {
    static_assert(MT % 2 == 0, "row tiles come in two halves");
    constexpr int HA = MT / 2;  // row tiles per half
    constexpr int KI = D / 32;  // 32-wide head-dim slices of the score products
    constexpr int NB = D / 16;  // 16-wide head-dim blocks of O
    constexpr int CPR = D / 8;  // 16-byte pieces per K or V row
    constexpr int CS = 32 * CPR;  // 16-byte pieces per chunk and operand
    constexpr int WR = 16 * MT;
    constexpr int NF = 2 * KI;         // K fragments (16 keys x 32 head dims) per chunk
    constexpr int SL1 = MT * NF;       // matrix-core slots of phase 1
    constexpr int SL2 = MT * NB + MT;  // matrix-core slots of phase 2
    constexpr int NWT = 8 * HA;        // weights per lane formed in each phase
    constexpr int SC = 4;              // phase-2 slots before the reference check
    // 1 KB loads per chunk: each operand's chunk is CS / 64 blocks.  With one
    // load per wave the first half of the waves moves K and the second half
    // V; with more, the first half moves both.  On each SIMD the wave of the
    // second half is the one that waits for the matrix cores (the older wave
    // wins them), so the issue work goes to the first.
    constexpr int LPS = CS / 64 * 2 / NW;
    static_assert(LPS >= 1 && (LPS == 1 || LPS % 2 == 0) && LPS * NW == CS / 64 * 2, "chunk blocks split evenly over the waves");
    constexpr int BPO = LPS == 1 ? 1 : LPS;  // blocks per operand and loading wave
    // Four LDS objects; object x holds K stage x and V stage x-1 (mod 4).
    // Step n reads K(n+1) and V(n), both in one object, and every direct
    // load still in flight then targets one of the other three: distinct
    // objects let the compiler see that the reads never wait for them.
    __shared__ u32x4 lds_x0[2 * CS], lds_x1[2 * CS], lds_x2[2 * CS], lds_x3[2 * CS];
    auto obj = [&](auto x) __attribute__((always_inline)) -> u32x4* {
        constexpr int i = decltype(x)::value & 3;
        if constexpr (i == 0) return lds_x0;
        else if constexpr (i == 1) return lds_x1;
        else if constexpr (i == 2) return lds_x2;
        else return lds_x3;
    };
    auto k_stage = [&](auto st) __attribute__((always_inline)) -> u32x4* { return obj(st); };
    auto v_stage = [&](auto st) __attribute__((always_inline)) -> u32x4* {
        return obj(IntC<decltype(st)::value + 1>{}) + CS;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int grp = lane >> 4;
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
    const int ks2 = Hkv * D * 2;
    const uint16_t* qb = q + (int64_t)b * P * qs + (int64_t)head * D;
    const char* kb = reinterpret_cast<const char*>(k + (int64_t)b * P * Hkv * D + (int64_t)g * D);
    const char* vb = reinterpret_cast<const char*>(v + (int64_t)b * P * Hkv * D + (int64_t)g * D);
    const int valid_bytes = (P - 1) * ks2 + D * 2;

    bf16x8 qB[MT][KI];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = iw + 16 * mt + col;
        const bool ok = row < P;
        const uint16_t* qp = qb + (int64_t)(ok ? row : 0) * qs + 8 * grp;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            u32x4 w = load16(qp + 32 * i, ok);
            if (c_log2 < 0.f) w ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            qB[mt][i] = as_bf16x8(w);
        }
    }
    const float cs = fmaxf(fabsf(c_log2), 1e-30f);
    const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    // K operand: lane (col, grp) of fragment j = 2i + t reads key row
    // 8(col/4) + col%4 + 4t of the chunk, head dims 32i + 8grp .. +7.
    int ka_byte[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int r = 8 * (col >> 2) + (col & 3);
        ka_byte[i] = 16 * (r * CPR + k_pos(r, 4 * i + grp, CPR));
    }
    // V transpose reads: lane (L, grp) names row 8grp + L/4 and the 8 bytes
    // of head dims 16e + 4(L%4) .. +3; it receives keys 8grp + 0..3 (+4 for
    // the second read) of head dim 16e + L.
    int vt_byte[NB];
    {
        const int L = lane & 15, m = L & 3;
        const int r = 8 * grp + (L >> 2);
#pragma unroll
        for (int e = 0; e < NB; ++e)
            vt_byte[e] = r * CPR * 16 + v_pos(r, 2 * e + (m >> 1), CPR) * 16 + 8 * (m & 1);
    }
    // Chunk fill: a wave of the first half moves BPO 1 KB blocks (64 lanes x
    // 16 bytes) of K and of V, blocks wave, wave + NW/2, ... (with one load
    // per wave: every wave moves block wave mod NW/2 of K or of V).  Lane l
    // of block blk lands in slot 64*blk + l and fetches the piece the
    // swizzle places there.
    int blk[BPO], k_off[BPO], v_off[BPO];
#pragma unroll
    for (int x = 0; x < BPO; ++x) {
        blk[x] = LPS == 1 ? wave % (NW / 2) : (wave % (NW / 2)) + (NW / 2) * x;
        const int slot = 64 * blk[x] + lane;
        const int r = slot / CPR, pos = slot % CPR;
        k_off[x] = r * ks2 + 16 * k_pos(r, pos, CPR);
        v_off[x] = r * ks2 + 16 * v_pos(r, pos, CPR);
    }
    const int kv_end = causal ? min(P, i0 + rows_wg) : P;
    // Chunks of the workgroup: [c_lo, c_hi); of this wave: [n0, n_end).
    const int c_lo = window > 0 ? max(0, i0 - window + 1) / 32 : 0;
    const int c_hi = (kv_end + 31) / 32;
    const int wave_last_row = min(iw + WR, P) - 1;
    const int lim = causal ? min(kv_end, wave_last_row + 1) : kv_end;
    const int n0 = window > 0 ? max(0, iw - window + 1) / 32 : 0;
    const int n_end = (lim + 31) / 32;
    const bool active = iw < P && n0 < n_end;
    // The step tests below are one unsigned range test each, on bounds fixed
    // here: the wave works in steps [a_lo, a_lo + a_span) (from the empty
    // chunk before its first one to its last one), and chunks
    // [u_lo, u_lo + u_span] need no mask (whole rows inside the prompt, below
    // the diagonal of every row of the wave and inside every row's window).
    const int a_lo = n0 - 1;
    const unsigned a_span = active ? (unsigned)max(0, min(n_end, c_hi) - a_lo) : 0u;
    int u_hi = (P - 32) >> 5;
    if (causal) u_hi = min(u_hi, (iw - 31) >> 5);
    int u_lo = window > 0 ? ((wave_last_row - window) >> 5) + 1 : -(1 << 28);
    if (u_hi < u_lo) u_lo = u_hi = 1 << 28;  // no such chunk
    const unsigned u_span = (unsigned)(u_hi - u_lo);
    // Start loading chunk c of K or V into stage `stage`.  Each load gets a
    // buffer resource based at the chunk's first row; rows at or past P, and
    // chunks before the first or past the workgroup's last one, read as zero
    // without touching memory.
    auto fill_k = [&](auto stage, int c) __attribute__((always_inline)) {
        if (wave >= NW / 2) return;
        const int base = 32 * min(max(c, 0), c_hi) * ks2;
        const int nrec = c >= 0 && c < c_hi ? valid_bytes - base : 0;
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb + base), (short)0, nrec, 0x00020000);
#pragma unroll
        for (int x = 0; x < BPO; ++x)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&k_stage(stage)[64 * blk[x]], 16u, (unsigned)k_off[x], 0u, 0u, 0u);
    };
    auto fill_v = [&](auto stage, int c) __attribute__((always_inline)) {
        if (LPS == 1 ? wave < NW / 2 : wave >= NW / 2) return;
        const int base = 32 * min(max(c, 0), c_hi) * ks2;
        const int nrec = c >= 0 && c < c_hi ? valid_bytes - base : 0;
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb + base), (short)0, nrec, 0x00020000);
#pragma unroll
        for (int x = 0; x < BPO; ++x)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&v_stage(stage)[64 * blk[x]], 16u, (unsigned)v_off[x], 0u, 0u, 0u);
    };

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

    // no row of the wave needs a mask in chunk n
    auto unmasked = [&](int n) __attribute__((always_inline)) -> bool {
        return (unsigned)(n - u_lo) <= u_span;
    };
    // Causal, window and tail mask of the chunk starting at key kc0.  Chunks
    // at or past n_end lie past every row's last key, so it removes them whole.
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
    auto max8 = [&](const f32x4 (&s)[2]) __attribute__((always_inline)) -> float {
        const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[0][0], s[0][1]), s[0][2]);
        const float bb = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[0][3], s[1][0]), s[1][1]);
        const float c = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[1][2], s[1][3]), a);
        return __builtin_elementwise_maximum(bb, c);
    };
    // Move row tile mt's reference maxima to the integer at or above the new
    // scores and rescale its accumulators by the exact power of two; returns
    // this lane's row factor.
    auto rescale = [&](int mt, const f32x4 (&s)[2]) __attribute__((always_inline)) -> float {
        const float mx = max8(s);
        float rm = fmaxf(mx, __shfl_xor(mx, 16));
        rm = fmaxf(rm, __shfl_xor(rm, 32));
        const float m_new = fmaxf(m_ref[mt], ceilf(rm * cs));
        const float alpha = __builtin_amdgcn_ldexpf(1.0f, (int)fmaxf(m_ref[mt] - m_new, -256.f));
        m_ref[mt] = m_new;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * grp + r);
            osum[mt][r] *= ar;
#pragma unroll
            for (int e = 0; e < NB; ++e) O[mt][e][r] *= ar;
        }
        return alpha;
    };
    // Keep a packed weight where it is formed: the optimiser would otherwise
    // sink its whole computation to its first use in the next phase, out of
    // the matrix-core stream it is meant to overlap.
    auto pin = [&](uint32_t& x) __attribute__((always_inline)) { asm volatile("" : "+v"(x)); };
    auto weight = [&](const f32x4 (&s)[2], float mr, int u) __attribute__((always_inline)) -> float {
        return fast_exp2(__builtin_fmaf(s[u >> 2][u & 3], cs, -mr));
    };
    auto kfrag = [&](const char* kl, int j) __attribute__((always_inline)) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(kl + ka_byte[j >> 1] + 4 * (j & 1) * CPR * 16);
    };
    auto vfrag = [&](const char* vl, int e) __attribute__((always_inline)) -> u32x4 {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + vt_byte[e]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + vt_byte[e] + 4 * CPR * 16));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };

    // Carried from one step to the next: scores of the upper half of the row
    // tiles and weights of the lower half, of the current chunk.  Before a
    // wave's first chunk they stand for an empty chunk (weights zero).
    f32x4 sB[HA][2];
    u32x4 pA[HA];
    u32x4 kf_next[2];
#pragma unroll
    for (int a = 0; a < HA; ++a) {
        sB[a][0] = sB[a][1] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
        pA[a] = u32x4{0u, 0u, 0u, 0u};
    }

    // Step n (V of chunk n in stage S, K of chunk n+1 in stage S+1): finish
    // chunk n (upper-half weights, P*V) and start chunk n+1 (scores,
    // lower-half weights).  Weight u of a phase belongs to row tile u / 8 of
    // the half, score u % 8 of the lane.
    auto step = [&](auto S, int n) __attribute__((always_inline)) {
        constexpr int s_v = decltype(S)::value;
        constexpr int s_k = (s_v + 1) & 3;
        // This wave's loads up to the ones two barriers back have landed
        // (K(n+2), V(n+1) and older; those of the previous barrier may still
        // fly); once every wave is here, they are visible to all, and nobody
        // reads K(n) or V(n-1) again.
        // The waits are explicit (vmcnt: the loads of one barrier may fly;
        // lgkmcnt(2)): a workgroup
        // fence would also wait for the direct loads still in flight.  The
        // two LDS reads allowed to fly are the last ones of the previous
        // step, its prefetch of K(n+1), which no load started here
        // overwrites; LDS reads complete in order, so every earlier read of
        // K(n) and V(n-1) has completed.  The wavefront-scope fences emit
        // nothing and only keep the compiler from moving LDS accesses across
        // the barrier.
        __builtin_amdgcn_s_waitcnt(0x0070 | (LPS == 1 ? 1 : 2 * LPS) | (2 << 8));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        fill_k(IntC<s_v>{}, n + 4);
        fill_v(IntC<(s_v + 3) & 3>{}, n + 3);
        const char* kl = reinterpret_cast<const char*>(k_stage(IntC<s_k>{}));
        // The first two K fragments of the next step (chunk n+2, complete and
        // visible since this barrier), read now so that step starts without
        // waiting for LDS.
        const char* kl_next = reinterpret_cast<const char*>(k_stage(IntC<(s_k + 1) & 3>{}));
        if (__builtin_expect((unsigned)(n - a_lo) >= a_span, 0)) {
            kf_next[0] = kfrag(kl_next, 0);
            kf_next[1] = kfrag(kl_next, 1);
            return;
        }
        const char* vl = reinterpret_cast<const char*>(v_stage(IntC<s_v>{}));
        u32x4 vf[NB];
        float w[NWT];
        // ---- phase 1: scores of chunk n+1 || upper-half weights of chunk n
        u32x4 kf[NF];
        kf[0] = kf_next[0];
        kf[1] = kf_next[1];
        float mB[HA];
#pragma unroll
        for (int a = 0; a < HA; ++a) mB[a] = m_ref[HA + a];
        f32x4 sn[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sn[mt][0] = sn[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 pB[HA];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            if (j + 2 < NF) kf[j + 2] = kfrag(kl, j + 2);
            if (j + 3 >= NF) vf[j + 3 - NF] = vfrag(vl, j + 3 - NF);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int sl = MT * j + mt;
                sn[mt][j & 1] = mfma16x16x32(as_bf16x8(kf[j]), qB[mt][j >> 1], sn[mt][j & 1]);
#pragma unroll
                for (int u = 0; u < NWT; ++u)
                    if (wslot(u, SL1, NWT) == sl) w[u] = weight(sB[u >> 3], mB[u >> 3], u & 7);
#pragma unroll
                for (int p = 0; p < 4 * HA; ++p)
                    if (wslot(2 * p + 1, SL1, NWT) + 1 == sl) {
                        uint32_t x = pack_bf16x2_rne(w[2 * p], w[2 * p + 1]);
                        pin(x);
                        pB[p >> 2][p & 3] = x;
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int p = 0; p < 4 * HA; ++p)
            if (wslot(2 * p + 1, SL1, NWT) + 1 >= SL1) pB[p >> 2][p & 3] = pack_bf16x2_rne(w[2 * p], w[2 * p + 1]);

        // ---- between phases: mask of chunk n+1 (rare: diagonal, window edges, tail)
        if (__builtin_expect(!unmasked(n + 1), 0)) mask(32 * (n + 1), sn);
        // ---- phase 2: P*V of chunk n || reference check of chunk n+1, then
        // lower-half weights of chunk n+1.  The first SC slots carry the
        // maxima of the new scores (long landed by then); the check follows.
        // A moving reference (rare) rescales O, the sums and the weights still
        // feeding this P*V by the same exact power of two: everything O holds
        // so far is relative to the old reference, so the sum stays consistent.
        float mx[MT];
        auto slot2 = [&](int sl) __attribute__((always_inline)) {
            if (sl < HA) {
                osum[sl] = mfma16x16x32(as_bf16x8(pA[sl]), ones, osum[sl]);
            } else if (sl >= HA + MT * NB) {
                const int a = sl - HA - MT * NB;
                osum[HA + a] = mfma16x16x32(as_bf16x8(pB[a]), ones, osum[HA + a]);
            } else {
                const int e = (sl - HA) / MT, mt = (sl - HA) % MT;
                if (mt == 0 && e + 3 < NB) vf[e + 3] = vfrag(vl, e + 3);
                O[mt][e] = mfma16x16x32(as_bf16x8(mt < HA ? pA[mt % HA] : pB[mt % HA]), as_bf16x8(vf[e]), O[mt][e]);
            }
        };
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = 0; sl < SC; ++sl) {
            slot2(sl);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (mt * SC / MT == sl) mx[mt] = max8(sn[mt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        bool gr = false;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) gr |= mx[mt] * cs > m_ref[mt] + kRescaleSlack;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(gr) != 0, 0)) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float alpha = rescale(mt, sn[mt]);
                u32x4& pw = mt < HA ? pA[mt % HA] : pB[mt % HA];
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    pw[p] = pack_bf16x2_rne(bf16_lo(pw[p]) * alpha, bf16_hi(pw[p]) * alpha);
            }
        }
        float mA[HA];
#pragma unroll
        for (int a = 0; a < HA; ++a) mA[a] = m_ref[a];
        u32x4 pn[HA];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = SC; sl < SL2; ++sl) {
            slot2(sl);
#pragma unroll
            for (int u = 0; u < NWT; ++u)
                if (SC + wslot(u, SL2 - SC, NWT) == sl) w[u] = weight(sn[u >> 3], mA[u >> 3], u & 7);
#pragma unroll
            for (int p = 0; p < 4 * HA; ++p)
                if (SC + wslot(2 * p + 1, SL2 - SC, NWT) + 1 == sl) {
                    uint32_t x = pack_bf16x2_rne(w[2 * p], w[2 * p + 1]);
                    pin(x);
                    pn[p >> 2][p & 3] = x;
                }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int p = 0; p < 4 * HA; ++p)
            if (SC + wslot(2 * p + 1, SL2 - SC, NWT) + 1 >= SL2) pn[p >> 2][p & 3] = pack_bf16x2_rne(w[2 * p], w[2 * p + 1]);
        kf_next[0] = kfrag(kl_next, 0);
        kf_next[1] = kfrag(kl_next, 1);
#pragma unroll
        for (int a = 0; a < HA; ++a) {
            pA[a] = pn[a];
            sB[a][0] = sn[HA + a][0];
            sB[a][1] = sn[HA + a][1];
        }
    };

    // Chunk c lives in stage (c - c_lo) mod 4.  The loop starts three steps
    // early: those steps only start the first loads (no wave has work before
    // step c_lo - 1), and they fill V(c_lo - 1), read by the empty chunk, with
    // real rows or zeros.  Every iteration runs four steps, so all loads come
    // from the same four places in the code and each step's waits hold by
    // construction; steps past c_hi - 1 only keep the barrier count even.
    for (int n = c_lo - 4; n < c_hi; n += 4) {
        step(IntC<0>{}, n);
        step(IntC<1>{}, n + 1);
        step(IntC<2>{}, n + 2);
        step(IntC<3>{}, n + 3);
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load may still target LDS at exit

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = iw + 16 * mt + 4 * grp + r;
            const float l = osum[mt][r];
            if (row < P) {
                uint16_t* dst = out + ((int64_t)b * P + row) * qs + (int64_t)head * D + col;
                const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
                for (int e = 0; e < NB; ++e) dst[16 * e] = (uint16_t)f32_to_bf16_rne(O[mt][e][r] * inv);
            }
        }
    }
}

template <int D, int MT, int NW>
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
    hipLaunchKernelGGL((prefill_bf16<D, MT, NW>), grid, block, 0, stream, q, k, v, P, Hq, Hkv, gsize, hw,
                       nbgh, nrb, causal ? 1 : 0, window, c_log2, out);
    return hipGetLastError() == hipSuccess;
}

inline bool launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int P,
                           int Hq, int Hkv, int d, bool causal, int window, float c_log2,
                           uint16_t* out, hipStream_t stream) {
    if (d == 128)
        return launch_prefill_cfg<128, kPrefillMT, kPrefillWaves>(q, k, v, B, P, Hq, Hkv, causal, window, c_log2, out, stream);
    return launch_prefill_cfg<64, kPrefillMT, kPrefillWaves>(q, k, v, B, P, Hq, Hkv, causal, window, c_log2, out, stream);
}

}  // namespace gqa
