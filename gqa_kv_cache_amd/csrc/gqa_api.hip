// libgqa: C ABI entry points (declared in include/gqa.h).
//
// Host side only: argument validation, split planning, workspace layout and
// kernel launches.  Every step of the computation runs in the HIP kernels
// included below.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <cstdlib>

#include "gqa.h"
#include "common.hpp"
#include "decode.hpp"
#include "decode_ex.hpp"
#include "prefill.hpp"

namespace {

constexpr int kMaxGroup = 64;
constexpr int64_t kMaxChunk = 8192;  // keys per automatic decode piece, at most
constexpr int64_t kMinChunkF32 = 256;  // keys per automatic fp32 decode piece, at least
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device, cached per device.
gqa_status current_cu_count(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cus = cached;
            return GQA_OK;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return GQA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return GQA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ----- debug check of the device-side lengths (GQA_CHECK_SEQLENS=1) ---------

bool check_lengths_requested() {
    const char* e = std::getenv("GQA_CHECK_SEQLENS");
    return e && e[0] == '1' && e[1] == '\0';
}

// Copies seqlens (and, with a block table, the table entries of every row a
// sequence holds) to the host on the caller's stream, waits for them and
// checks lo <= seqlens[b] <= Lmax and 0 <= entry < num_blocks.  Goes through
// a fixed buffer on the stack, so it allocates nothing.  Skipped while the
// stream is being captured into a graph, where nothing may wait.
gqa_status check_lengths(hipStream_t hs, const int32_t* seqlens, int B, int lo, int Lmax,
                         const int32_t* block_table, int max_blocks, int block_size,
                         int num_blocks) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(hs, &cap) != hipSuccess) return GQA_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return GQA_OK;
    constexpr int kBuf = 1024;
    int32_t len[kBuf], ent[kBuf];
    for (int b0 = 0; b0 < B; b0 += kBuf) {
        const int nb = B - b0 < kBuf ? B - b0 : kBuf;
        if (hipMemcpyAsync(len, seqlens + b0, sizeof(int32_t) * nb, hipMemcpyDeviceToHost, hs) != hipSuccess ||
            hipStreamSynchronize(hs) != hipSuccess)
            return GQA_ERR_HIP;
        for (int i = 0; i < nb; ++i) {
            if (len[i] < lo || len[i] > Lmax) return GQA_ERR_SHAPE;
            if (!block_table) continue;
            const int used = (len[i] + block_size - 1) / block_size;  // blocks holding rows < len
            const int32_t* row = block_table + (int64_t)(b0 + i) * max_blocks;
            for (int e0 = 0; e0 < used; e0 += kBuf) {
                const int ne = used - e0 < kBuf ? used - e0 : kBuf;
                if (hipMemcpyAsync(ent, row + e0, sizeof(int32_t) * ne, hipMemcpyDeviceToHost, hs) != hipSuccess ||
                    hipStreamSynchronize(hs) != hipSuccess)
                    return GQA_ERR_HIP;
                for (int k = 0; k < ne; ++k)
                    if (ent[k] < 0 || ent[k] >= num_blocks) return GQA_ERR_SHAPE;
            }
        }
    }
    return GQA_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct DecodePlan {
    int splits;  // pieces the cached length is cut into
    int chunk;   // keys per piece
};

gqa_status check_heads(int Hq, int Hkv, int d) {
    if (Hq <= 0 || Hkv <= 0) return GQA_ERR_SHAPE;
    if (Hq % Hkv != 0) return GQA_ERR_GROUP;
    if (d != 64 && d != 128) return GQA_ERR_HEADDIM;
    if (Hq / Hkv > kMaxGroup) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

gqa_status plan_decode(int B, int Hq, int Hkv, int d, int Lmax, gqa_dtype dtype, int num_splits,
                       DecodePlan* plan) {
    if (B <= 0 || Lmax <= 0) return GQA_ERR_SHAPE;
    gqa_status st = check_heads(Hq, Hkv, d);
    if (st != GQA_OK) return st;
    if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_DTYPE;
    if (num_splits < 0 || num_splits > Lmax) return GQA_ERR_UNSUPPORTED;
    // byte offsets inside one sequence's cache slice are 32-bit
    if ((int64_t)(Lmax + gqa::kDecodeStep) * Hkv * d * 4 > INT_MAX) return GQA_ERR_SHAPE;
    int64_t chunk;
    if (num_splits == 0) {
        // One workgroup per (sequence, KV head) streams the whole cached
        // length when that already gives every compute unit a workgroup;
        // otherwise cut the length so it does.  Pieces are capped at
        // kMaxChunk keys so ragged batches stay balanced.
        int cus = 0;
        st = current_cu_count(&cus);
        if (st != GQA_OK) return st;
        const int64_t pairs = (int64_t)B * Hkv;
        int64_t splits = cdiv(cus, pairs);
        // fp32 pieces hold at least kMinChunkF32 keys: below that the fixed
        // cost of a piece and of the merge outweighs the parallelism
        if (dtype == GQA_F32 && splits > cdiv(Lmax, kMinChunkF32)) splits = cdiv(Lmax, kMinChunkF32);
        if (splits < cdiv(Lmax, kMaxChunk)) splits = cdiv(Lmax, kMaxChunk);
        chunk = cdiv(cdiv(Lmax, splits), gqa::kDecodeStep) * gqa::kDecodeStep;
    } else {
        chunk = cdiv(Lmax, num_splits);
    }
    const int64_t splits = cdiv(Lmax, chunk);
    if ((int64_t)B * Hkv * splits > INT_MAX) return GQA_ERR_SHAPE;
    plan->splits = (int)splits;
    plan->chunk = (int)chunk;
    return GQA_OK;
}

// Workspace: acc [B, Hq, splits, d] fp32, then (m, l) [B, Hq, splits, 2] fp32.
size_t workspace_acc_bytes(int B, int Hq, int d, int splits) {
    return (size_t)B * Hq * splits * d * sizeof(float);
}
size_t workspace_bytes_for(int B, int Hq, int d, int splits) {
    if (splits <= 1) return 0;
    return workspace_acc_bytes(B, Hq, d, splits) + (size_t)B * Hq * splits * 2 * sizeof(float);
}

template <int D>
void launch_split_bf16(int nt, dim3 grid, hipStream_t st, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const int32_t* sl, int Hq, int Hkv, int Lmax, int gs, int S,
                       int chunk, float c, uint16_t* out, float* wa, float* wm) {
    dim3 block(gqa::kDecodeThreads);
    switch (nt) {
        case 1: hipLaunchKernelGGL((gqa::decode_split_bf16<D, 1>), grid, block, 0, st, q, k, v, sl, Hq, Hkv, Lmax, gs, S, chunk, c, out, wa, wm); break;
        case 2: hipLaunchKernelGGL((gqa::decode_split_bf16<D, 2>), grid, block, 0, st, q, k, v, sl, Hq, Hkv, Lmax, gs, S, chunk, c, out, wa, wm); break;
        case 3: hipLaunchKernelGGL((gqa::decode_split_bf16<D, 3>), grid, block, 0, st, q, k, v, sl, Hq, Hkv, Lmax, gs, S, chunk, c, out, wa, wm); break;
        // Four tiles.  Short pieces: one tile per wave, so no partial sums
        // are combined across waves (the combine would dominate).  Pieces of
        // 512 keys or more: the waves split the keys as for fewer tiles,
        // which reads each row once instead of once per tile (about 10%
        // faster for 64-head groups at 512-1024-key pieces).
        default:
            if (chunk >= 512)
                hipLaunchKernelGGL((gqa::decode_split_bf16<D, 4>), grid, block, 0, st, q, k, v, sl, Hq, Hkv, Lmax, gs, S, chunk, c, out, wa, wm);
            else
                hipLaunchKernelGGL((gqa::decode_split_bf16_tiles<D>), grid, block, 0, st, q, k, v, sl, Hq, Hkv, Lmax, gs, S, chunk, c, out, wa, wm);
            break;
    }
}

// ----- extended decode ------------------------------------------------------

struct ExPlan {
    int splits, chunk, elt;
    size_t ws_bytes;
};

gqa_status plan_decode_ex(const gqa_decode_ex_args* a, bool query_device, ExPlan* plan) {
    if (a->B <= 0 || a->T <= 0 || a->Lmax <= 0 || a->window < 0) return GQA_ERR_SHAPE;
    gqa_status st = check_heads(a->Hq, a->Hkv, a->d);
    if (st != GQA_OK) return st;
    if (a->dtype != GQA_BF16) return GQA_ERR_DTYPE;
    if (a->kv_dtype != GQA_BF16 && a->kv_dtype != GQA_FP8_E4M3 && a->kv_dtype != GQA_FP8_E5M2) return GQA_ERR_DTYPE;
    if ((int64_t)a->T * (a->Hq / a->Hkv) > kMaxGroup) return GQA_ERR_UNSUPPORTED;
    if (a->block_table) {
        if (a->block_size < 16 || a->block_size % 16 != 0 || a->max_blocks <= 0 || a->num_blocks <= 0)
            return GQA_ERR_SHAPE;
        if ((int64_t)a->max_blocks * a->block_size != a->Lmax) return GQA_ERR_SHAPE;
    }
    if (a->num_splits < 0 || a->num_splits > a->Lmax) return GQA_ERR_UNSUPPORTED;
    // the rows of one 32-key step are addressed with 32-bit byte offsets
    const int64_t elt = a->kv_dtype == GQA_BF16 ? 2 : 1;
    if ((int64_t)gqa::kDecodeStep * a->Hkv * a->d * elt > INT_MAX) return GQA_ERR_SHAPE;
    int64_t chunk;
    if (a->num_splits == 0) {
        int cus = 0;
        if (query_device) {
            st = current_cu_count(&cus);
            if (st != GQA_OK) return st;
        } else {
            cus = 256;
        }
        const int64_t pairs = (int64_t)a->B * a->Hkv;
        int64_t splits = cdiv(cus, pairs);
        if (splits < cdiv(a->Lmax, kMaxChunk)) splits = cdiv(a->Lmax, kMaxChunk);
        chunk = cdiv(a->Lmax, splits);
    } else {
        chunk = cdiv(a->Lmax, a->num_splits);
    }
    // pieces start on 32-key steps, so a step never crosses a cache block
    chunk = cdiv(chunk, gqa::kDecodeStep) * gqa::kDecodeStep;
    const int64_t splits = cdiv(a->Lmax, chunk);
    const int64_t rows = (int64_t)a->B * a->T * a->Hq;
    if ((int64_t)a->B * a->Hkv * splits > INT_MAX || rows > INT_MAX) return GQA_ERR_SHAPE;
    plan->splits = (int)splits;
    plan->chunk = (int)chunk;
    plan->elt = (int)elt;
    plan->ws_bytes = splits > 1 ? (size_t)rows * splits * (a->d + 2) * sizeof(float) : 0;
    return GQA_OK;
}

// Waves per workgroup of the extended kernel: an FP8 step moves half the
// bytes of a bf16 step, so twice the waves keep as many bytes in flight
// (up to 32 query rows; more rows need more registers than 8 waves allow).
template <bool KV8, int NT> constexpr int ex_waves() { return KV8 && NT <= 2 ? 8 : 4; }

template <int D, int KV, bool H16>
void launch_decode_ex(int nt, dim3 grid, hipStream_t hs, const gqa_decode_ex_args* a, const ExPlan& p,
                      float c, float* wa, float* wm) {
    dim3 block;
    auto q = static_cast<const uint16_t*>(a->q);
    auto k = static_cast<uint8_t*>(a->k_cache);
    auto v = static_cast<uint8_t*>(a->v_cache);
    auto kn = static_cast<const uint8_t*>(a->k_new);
    auto vn = static_cast<const uint8_t*>(a->v_new);
    auto o = static_cast<uint16_t*>(a->out);
    const int gs = a->Hq / a->Hkv;
#define GQA_EX_ARGS q, k, v, a->seqlens, a->k_scale, a->v_scale, a->block_table, a->max_blocks, \
                    a->block_size, a->num_blocks, kn, vn, a->T, a->Hq, a->Hkv, a->Lmax, gs, p.splits, \
                    p.chunk, a->window, c, o, wa, wm
#define GQA_EX_CASE(N) block = dim3(64 * ex_waves<KV != 0, N>()); \
    hipLaunchKernelGGL((gqa::decode_ex_kernel<D, N, KV, ex_waves<KV != 0, N>(), H16>), grid, block, 0, hs, GQA_EX_ARGS)
    switch (nt) {
        case 1: GQA_EX_CASE(1); break;
        case 2: GQA_EX_CASE(2); break;
        case 3: GQA_EX_CASE(3); break;
        default: GQA_EX_CASE(4); break;
    }
#undef GQA_EX_CASE
#undef GQA_EX_ARGS
}

// Cache format and block shape -> kernel.  H16: paged blocks of a 16-row
// multiple that is not a 32-row one, so a 32-key step may span two blocks.
template <int D>
void launch_decode_ex_for(int nt, dim3 grid, hipStream_t hs, const gqa_decode_ex_args* a, const ExPlan& p,
                          float c, float* wa, float* wm) {
    const bool h16 = a->block_table != nullptr && a->block_size % 32 != 0;
    if (a->kv_dtype == GQA_FP8_E4M3) {
        if (h16) launch_decode_ex<D, 1, true>(nt, grid, hs, a, p, c, wa, wm);
        else launch_decode_ex<D, 1, false>(nt, grid, hs, a, p, c, wa, wm);
    } else if (a->kv_dtype == GQA_FP8_E5M2) {
        if (h16) launch_decode_ex<D, 2, true>(nt, grid, hs, a, p, c, wa, wm);
        else launch_decode_ex<D, 2, false>(nt, grid, hs, a, p, c, wa, wm);
    } else {
        if (h16) launch_decode_ex<D, 0, true>(nt, grid, hs, a, p, c, wa, wm);
        else launch_decode_ex<D, 0, false>(nt, grid, hs, a, p, c, wa, wm);
    }
}

gqa_status validate_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seqlens, int B, int Hq, int Hkv, int d, int Lmax,
                           gqa_dtype dtype, const void* out, int num_splits, DecodePlan* plan);
gqa_status run_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, int B, int Hq, int Hkv, int d, int Lmax, float scale,
                      gqa_dtype dtype, void* out, void* workspace, const DecodePlan& plan,
                      void* stream);

// ----- static scratch of gqa_decode_noalloc (the array itself is below) -----
constexpr size_t kScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

// The split partials of gqa_decode_noalloc live in this array instead of a
// caller buffer.  Every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names a host
// stand-in, never the device memory: kernels and copies get the address
// hipGetSymbolAddress returns for the current device, cached per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

gqa_status scratch_address(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        // Resolving the symbol twice from racing threads is harmless: both
        // get the same address.
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GQA_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return GQA_OK;
}

}  // namespace

extern "C" {

const char* gqa_status_str(gqa_status s) {
    switch (s) {
        case GQA_OK: return "GQA_OK";
        case GQA_ERR_NULL: return "GQA_ERR_NULL: a required pointer is NULL";
        case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE: a size is out of range";
        case GQA_ERR_GROUP: return "GQA_ERR_GROUP: Hq is not a multiple of Hkv";
        case GQA_ERR_HEADDIM: return "GQA_ERR_HEADDIM: head dim must be 64 or 128";
        case GQA_ERR_DTYPE: return "GQA_ERR_DTYPE: dtype not supported by this call";
        case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN: a data pointer is not 16-byte aligned";
        case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
        case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: group size above 64 or num_splits out of range";
        case GQA_ERR_HIP: return "GQA_ERR_HIP: the HIP runtime reported an error";
        case GQA_ERR_SCRATCH_LIMIT: return "GQA_ERR_SCRATCH_LIMIT: the split partials exceed the static scratch of gqa_decode_noalloc";
    }
    return "GQA status: unknown code";
}

gqa_status gqa_decode_num_splits(int B, int Hq, int Hkv, int d, int Lmax, gqa_dtype dtype,
                                 int num_splits, int* splits) {
    if (!splits) return GQA_ERR_NULL;
    DecodePlan plan;
    gqa_status st = plan_decode(B, Hq, Hkv, d, Lmax, dtype, num_splits, &plan);
    if (st != GQA_OK) return st;
    *splits = plan.splits;
    return GQA_OK;
}

gqa_status gqa_decode_workspace_size(int B, int Hq, int Hkv, int d, int Lmax, gqa_dtype dtype,
                                     int num_splits, size_t* bytes) {
    if (!bytes) return GQA_ERR_NULL;
    DecodePlan plan;
    gqa_status st = plan_decode(B, Hq, Hkv, d, Lmax, dtype, num_splits, &plan);
    if (st != GQA_OK) return st;
    *bytes = workspace_bytes_for(B, Hq, d, plan.splits);
    return GQA_OK;
}

gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, int B, int Hq, int Hkv, int d, int Lmax, float scale,
                      gqa_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                      int num_splits, void* stream) {
    DecodePlan plan;
    gqa_status st = validate_decode(q, k_cache, v_cache, seqlens, B, Hq, Hkv, d, Lmax, dtype, out,
                                    num_splits, &plan);
    if (st != GQA_OK) return st;
    const size_t need = workspace_bytes_for(B, Hq, d, plan.splits);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return GQA_ERR_WORKSPACE;
    return run_decode(q, k_cache, v_cache, seqlens, B, Hq, Hkv, d, Lmax, scale, dtype, out,
                      need ? workspace : nullptr, plan, stream);
}

gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seqlens, int B, int Hq, int Hkv, int d, int Lmax,
                              float scale, gqa_dtype dtype, void* out, int num_splits,
                              void* stream) {
    DecodePlan plan;
    gqa_status st = validate_decode(q, k_cache, v_cache, seqlens, B, Hq, Hkv, d, Lmax, dtype, out,
                                    num_splits, &plan);
    if (st != GQA_OK) return st;
    const size_t need = workspace_bytes_for(B, Hq, d, plan.splits);
    if (need > kScratchBytes) return GQA_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != GQA_OK) return st;
    }
    return run_decode(q, k_cache, v_cache, seqlens, B, Hq, Hkv, d, Lmax, scale, dtype, out, ws,
                      plan, stream);
}

}  // extern "C"

namespace {

// Argument checks shared by the two decode entry points, then the plan.
gqa_status validate_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seqlens, int B, int Hq, int Hkv, int d, int Lmax,
                           gqa_dtype dtype, const void* out, int num_splits, DecodePlan* plan) {
    if (!q || !k_cache || !v_cache || !seqlens || !out) return GQA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return GQA_ERR_ALIGN;
    // Validate sizes before touching the runtime.
    if (B <= 0 || Lmax <= 0) return GQA_ERR_SHAPE;
    gqa_status st = check_heads(Hq, Hkv, d);
    if (st != GQA_OK) return st;
    if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_DTYPE;
    if (num_splits < 0 || num_splits > Lmax) return GQA_ERR_UNSUPPORTED;
    // queries the device only when num_splits == 0
    return plan_decode(B, Hq, Hkv, d, Lmax, dtype, num_splits, plan);
}

// Launches of one decode call on a validated plan; `workspace` holds the
// split partials (NULL when the plan has one piece).
gqa_status run_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, int B, int Hq, int Hkv, int d, int Lmax, float scale,
                      gqa_dtype dtype, void* out, void* workspace, const DecodePlan& plan,
                      void* stream) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (check_lengths_requested()) {
        const gqa_status st = check_lengths(hs, seqlens, B, 0, Lmax, nullptr, 0, 1, 0);
        if (st != GQA_OK) return st;
    }
    const int gs = Hq / Hkv;
    const int S = plan.splits;
    const float c = scale * gqa::kLog2e;
    float* ws_acc = S > 1 ? static_cast<float*>(workspace) : nullptr;
    float* ws_ml = S > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    workspace_acc_bytes(B, Hq, d, S))
                         : nullptr;
    dim3 grid((unsigned)((int64_t)B * Hkv * S));

    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (dtype == GQA_BF16) {
        const int nt = (gs + 15) / 16;
        auto qp = static_cast<const uint16_t*>(q);
        auto kp = static_cast<const uint16_t*>(k_cache);
        auto vp = static_cast<const uint16_t*>(v_cache);
        auto op = static_cast<uint16_t*>(out);
        if (d == 128)
            launch_split_bf16<128>(nt, grid, hs, qp, kp, vp, seqlens, Hq, Hkv, Lmax, gs, S, plan.chunk, c, op, ws_acc, ws_ml);
        else
            launch_split_bf16<64>(nt, grid, hs, qp, kp, vp, seqlens, Hq, Hkv, Lmax, gs, S, plan.chunk, c, op, ws_acc, ws_ml);
    } else {
        auto qp = static_cast<const float*>(q);
        auto kp = static_cast<const float*>(k_cache);
        auto vp = static_cast<const float*>(v_cache);
        auto op = static_cast<float*>(out);
        dim3 block(gqa::kDecodeThreads);
        if (d == 128)
            hipLaunchKernelGGL((gqa::decode_split_f32<128>), grid, block, 0, hs, qp, kp, vp, seqlens, Hq, Hkv, Lmax, gs, S, plan.chunk, c, op, ws_acc, ws_ml);
        else
            hipLaunchKernelGGL((gqa::decode_split_f32<64>), grid, block, 0, hs, qp, kp, vp, seqlens, Hq, Hkv, Lmax, gs, S, plan.chunk, c, op, ws_acc, ws_ml);
    }
    if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
    if (S > 1) {
        dim3 mgrid((unsigned)((int64_t)B * Hq));
        dim3 mblock(64);
        if (dtype == GQA_BF16) {
            if (d == 128)
                hipLaunchKernelGGL((gqa::decode_merge<128, true>), mgrid, mblock, 0, hs, ws_acc, ws_ml, seqlens, Hq, Lmax, S, plan.chunk, out);
            else
                hipLaunchKernelGGL((gqa::decode_merge<64, true>), mgrid, mblock, 0, hs, ws_acc, ws_ml, seqlens, Hq, Lmax, S, plan.chunk, out);
        } else {
            if (d == 128)
                hipLaunchKernelGGL((gqa::decode_merge<128, false>), mgrid, mblock, 0, hs, ws_acc, ws_ml, seqlens, Hq, Lmax, S, plan.chunk, out);
            else
                hipLaunchKernelGGL((gqa::decode_merge<64, false>), mgrid, mblock, 0, hs, ws_acc, ws_ml, seqlens, Hq, Lmax, S, plan.chunk, out);
        }
        if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
    }
    return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_decode_ex_workspace_size(const gqa_decode_ex_args* a, size_t* bytes) {
    if (!a || !bytes) return GQA_ERR_NULL;
    ExPlan plan;
    gqa_status st = plan_decode_ex(a, true, &plan);
    if (st != GQA_OK) return st;
    *bytes = plan.ws_bytes;
    return GQA_OK;
}

gqa_status gqa_decode_ex(const gqa_decode_ex_args* a, void* stream) {
    if (!a) return GQA_ERR_NULL;
    if (!a->q || !a->k_cache || !a->v_cache || !a->seqlens || !a->out) return GQA_ERR_NULL;
    if ((a->k_new == nullptr) != (a->v_new == nullptr)) return GQA_ERR_NULL;
    const bool kv_fp8 = a->kv_dtype == GQA_FP8_E4M3 || a->kv_dtype == GQA_FP8_E5M2;
    if (kv_fp8 && (!a->k_scale || !a->v_scale)) return GQA_ERR_NULL;
    if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || !aligned16(a->out))
        return GQA_ERR_ALIGN;
    if (a->k_new && (!aligned16(a->k_new) || !aligned16(a->v_new))) return GQA_ERR_ALIGN;
    // validate everything before the first device query
    ExPlan plan;
    gqa_status st = plan_decode_ex(a, false, &plan);
    if (st != GQA_OK) return st;
    st = plan_decode_ex(a, true, &plan);
    if (st != GQA_OK) return st;
    if (plan.ws_bytes > 0 && (!a->workspace || a->workspace_bytes < plan.ws_bytes || !aligned16(a->workspace)))
        return GQA_ERR_WORKSPACE;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (check_lengths_requested()) {
        st = check_lengths(hs, a->seqlens, a->B, a->T, a->Lmax, a->block_table, a->max_blocks,
                           a->block_size, a->num_blocks);
        if (st != GQA_OK) return st;
    }
    const int S = plan.splits;
    const int64_t rows = (int64_t)a->B * a->T * a->Hq;
    float* ws_acc = plan.ws_bytes ? static_cast<float*>(a->workspace) : nullptr;
    float* ws_ml = plan.ws_bytes ? ws_acc + rows * S * a->d : nullptr;
    (void)hipGetLastError();
    const int nt = (a->T * (a->Hq / a->Hkv) + 15) / 16;
    const float c = a->scale * gqa::kLog2e;
    dim3 grid((unsigned)((int64_t)a->B * a->Hkv * S));
    if (a->d == 128) launch_decode_ex_for<128>(nt, grid, hs, a, plan, c, ws_acc, ws_ml);
    else launch_decode_ex_for<64>(nt, grid, hs, a, plan, c, ws_acc, ws_ml);
    if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
    if (S > 1) {
        dim3 mgrid((unsigned)rows);
        auto o = static_cast<uint16_t*>(a->out);
        if (a->d == 128)
            hipLaunchKernelGGL((gqa::decode_ex_merge<128>), mgrid, dim3(64), 0, hs, ws_acc, ws_ml, a->seqlens, a->T, a->Hq, a->Lmax, S, plan.chunk, a->window, o);
        else
            hipLaunchKernelGGL((gqa::decode_ex_merge<64>), mgrid, dim3(64), 0, hs, ws_acc, ws_ml, a->seqlens, a->T, a->Hq, a->Lmax, S, plan.chunk, a->window, o);
        if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
    }
    return GQA_OK;
}

gqa_status gqa_prefill_ex(const void* q, const void* k, const void* v, int B, int P, int Hq,
                          int Hkv, int d, int causal, int window, float scale, gqa_dtype dtype,
                          void* out, void* stream) {
    if (!q || !k || !v || !out) return GQA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_ALIGN;
    if (B <= 0 || P <= 0 || window < 0) return GQA_ERR_SHAPE;
    gqa_status st = check_heads(Hq, Hkv, d);
    if (st != GQA_OK) return st;
    if (dtype != GQA_BF16) return GQA_ERR_DTYPE;
    if (window > 0 && !causal) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq * cdiv(P, gqa::kPrefillRows) > INT_MAX) return GQA_ERR_SHAPE;
    // byte offsets inside one sequence's K/V are 32-bit
    if ((int64_t)(P + (4 * gqa::kPrefillChunk)) * Hkv * d * 2 > INT_MAX) return GQA_ERR_SHAPE;
    (void)hipGetLastError();
    if (!gqa::launch_prefill(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                             static_cast<const uint16_t*>(v), B, P, Hq, Hkv, d, causal != 0, window,
                             scale * gqa::kLog2e, static_cast<uint16_t*>(out),
                             static_cast<hipStream_t>(stream)))
        return GQA_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
    return GQA_OK;
}

gqa_status gqa_prefill(const void* q, const void* k, const void* v, int B, int P, int Hq, int Hkv,
                       int d, int causal, float scale, gqa_dtype dtype, void* out, void* stream) {
    return gqa_prefill_ex(q, k, v, B, P, Hq, Hkv, d, causal, 0, scale, dtype, out, stream);
}

uint64_t gqa_kv_cache_elems(uint64_t L, uint64_t Hkv, uint64_t d) { return 2ull * L * Hkv * d; }

uint64_t gqa_decode_bytes(const int32_t* host_seqlens, int B, int Hq, int Hkv, int d,
                          gqa_dtype dtype) {
    const uint64_t elt = dtype == GQA_BF16 ? 2 : dtype == GQA_F32 ? 4 : 0;
    if (!elt || !host_seqlens || B <= 0) return 0;
    uint64_t rows = 0;
    for (int b = 0; b < B; ++b) rows += host_seqlens[b] > 0 ? (uint64_t)host_seqlens[b] : 0;
    const uint64_t kv = rows * gqa_kv_cache_elems(1, (uint64_t)Hkv, (uint64_t)d) * elt;
    const uint64_t q_and_out = 2ull * (uint64_t)B * Hq * d * elt;
    return kv + q_and_out;
}

uint64_t gqa_decode_flops(const int32_t* host_seqlens, int B, int Hq, int d) {
    if (!host_seqlens || B <= 0) return 0;
    uint64_t rows = 0;
    for (int b = 0; b < B; ++b) rows += host_seqlens[b] > 0 ? (uint64_t)host_seqlens[b] : 0;
    return 4ull * (uint64_t)Hq * (uint64_t)d * rows;
}

uint64_t gqa_prefill_flops(int B, int P, int Hq, int d, int causal) {
    if (B <= 0 || P <= 0) return 0;
    const uint64_t p = (uint64_t)P;
    const uint64_t pairs = causal ? p * (p + 1) / 2 : p * p;
    return 4ull * (uint64_t)B * Hq * d * pairs;
}

uint64_t gqa_prefill_bytes(int B, int P, int Hq, int Hkv, int d, gqa_dtype dtype) {
    const uint64_t elt = dtype == GQA_BF16 ? 2 : dtype == GQA_F32 ? 4 : 0;
    if (B <= 0 || P <= 0) return 0;
    return (uint64_t)B * P * d * elt * (2ull * Hq + 2ull * Hkv);
}

}  // extern "C"
