// Fine stage of gated, tile-sparse video attention on gfx950: block-sparse
// online-softmax attention over the kept tiles, with the gated coarse term and
// the scatter back to natural token order fused into the epilogue.
//
// Method: SnackOnAI analysis of ComfyUI-Ref2VA-VSA, "The Code, Annotated",
// snippet two -- prefix key tiles are always kept (sink blocks [0, P)), prefix
// query tiles attend densely (sink queries [0, P)), block_len keeps padding
// out of the softmax, scale = D^-1/2, and the gate enters as the coarse-gate
// input; "It In Action", step three: each video query tile sees the prefix
// tiles plus its kept video tiles.
//
// Design (CDNA4):
//  - One wavefront per (head, 64 query rows of a tile). The wave holds the 64
//    query rows as MFMA B-operand fragments for the whole key list, so the
//    K/V of a key tile is consumed by exactly one wave and never has to be
//    shared through LDS: K and V arrive from L2/HBM as fully coalesced 1 KB
//    fragments (the layout written by the coarse stage) straight into VGPRs.
//  - S^T = K . Q^T and O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with fp32
//    accumulation. With keys as rows of S^T, each lane owns one query column,
//    so the running max / sum and the O rescale are per lane (plus one
//    cross-half exchange), and the S accumulator already has the register
//    layout of the P^T operand of the second product.
//  - The next key tile's K is fetched while P.V of the current one runs, and
//    the current V while S is computed (register double buffering).
//  - Heavy work first: prefix query tiles (dense over all n_t tiles) are
//    dispatched before the video query tiles (prefix + k tiles).
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "device.h"

namespace vsa {
namespace {

struct FineArgs {
    const uint16_t *q;          // [S][H][D]
    const uint16_t *kt;         // tiled K fragments [H][n_t][B/64][D/8][64][8]
    const uint16_t *vt;         // tiled V fragments
    const int32_t *row_src;     // [S_pad]
    const int32_t *block_len;   // [n_t]
    const int32_t *keep;        // [H][n_v][k]
    const float *o_coarse;      // [H][n_t][D]
    const uint16_t *gate;       // [S][H*D]
    uint16_t *out;              // [S][H][D]
    int H, P, n_v, n_t, k;
    float scale_log2e;
};

__device__ __forceinline__ bf16x8_t load_frag(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8_t *>(p);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((address_space(4))) const int32_t cint32_t;

__device__ __forceinline__ const cint32_t *to_const(const int32_t *p)
{
    return reinterpret_cast<const cint32_t *>(reinterpret_cast<uintptr_t>(p));
}
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Word 3 of a raw buffer resource (32-bit data format) for gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
constexpr float kLazy = 8.0f;  // log2-domain slack before the running max moves

template <int D, int B>
__global__ __launch_bounds__(64) void fine_attn_kernel(FineArgs a)
{
    constexpr int SUB = B / 64;   // 64-row blocks per tile
    constexpr int NC = D / 16;    // reduction chunks of S = K.Q^T
    constexpr int DB = D / 32;    // 32-row blocks of O^T (over d)
    constexpr int FR = D / 8;     // 1 KB fragments per 64-row block
    constexpr int HPU = 2 * SUB;  // 32-key halves per key tile
    const int lane = threadIdx.x;
    const int l32 = lane & 31, half = lane >> 5;

    // ---- work item: prefix query tiles first (heavy), then video query tiles.
    const int item = blockIdx.x;
    const int prefix_items = a.H * a.P * SUB;
    int h, tile, qsub;
    if (item < prefix_items) {
        h = item / (a.P * SUB);
        const int r = item % (a.P * SUB);
        tile = r / SUB;
        qsub = r % SUB;
    } else {
        const int it = item - prefix_items;
        h = it / (a.n_v * SUB);
        const int r = it % (a.n_v * SUB);
        tile = a.P + r / SUB;
        qsub = r % SUB;
    }
    const bool dense = tile < a.P;
    const int n_key_tiles = dense ? a.n_t : a.P + a.k;

    // ---- query fragments (B operand of S^T = K . Q^T): lane -> query 32qb + l32,
    // reduction slot e of chunk c -> d = 16c + 8*half + e. They are staged once
    // in LDS (16 KB per wave) and re-read for every S product, which keeps their
    // 64 VGPRs free for the K/V stream.
    __shared__ __attribute__((aligned(16))) bf16x8_t q_lds[2][NC][kWave];
    int tok[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        tok[qb] = a.row_src[size_t(tile) * B + 64 * qsub + 32 * qb + l32];
        const uint16_t *qrow = a.q + (size_t(tok[qb] < 0 ? 0 : tok[qb]) * a.H + h) * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8_t v = load_frag(qrow + 16 * c);
            if (tok[qb] < 0) v = bf16x8_t{};
            q_lds[qb][c][lane] = v;
        }
    }
    __syncthreads();

    // ---- key list. Kept tiles come from the coarse stage; clamping only guards
    // against a foreign keep list. The list and block_len are read-only and read
    // at wave-uniform addresses, so they go through the constant address space:
    // scalar loads, whose waits do not drain the in-flight K/V vector loads.
    const cint32_t *keep_s =
        to_const(dense ? a.keep : a.keep + (size_t(h) * a.n_v + (tile - a.P)) * a.k);
    const cint32_t *bl_s = to_const(a.block_len);
    auto half_tile = [&](int v) -> int {
        const int n = v / HPU;
        return (dense || n < a.P) ? n : min(max(keep_s[n - a.P], 0), a.n_t - 1);
    };

    // ---- K/V stream: one buffer resource per head (SGPRs); a fragment is read
    // with an SGPR byte offset plus the lane's 16-byte slot, fully coalesced.
    // Reads outside the head's region return zero instead of faulting.
    const uint32_t head_bytes = uint32_t(a.n_t) * B * D * 2;
    const size_t head_elems = size_t(h) * a.n_t * B * D;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)(a.kt + head_elems), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void *)(a.vt + head_elems), (short)0, head_bytes, kRsrcWord3);
    const int vlane = lane * 16;
    // Half v covers rows 32*(v % 2) .. +31 of 64-row block (v % HPU) / 2 of its tile.
    auto half_base = [&](int v) -> uint32_t {
        const int u = v % HPU;
        return (uint32_t(half_tile(v)) * SUB + uint32_t(u >> 1)) * FR * 1024u;
    };
    auto load_k = [&](int v, bf16x8_t (&Kb)[NC]) {
        const uint32_t base = half_base(v) + uint32_t(v & 1) * NC * 1024u;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            Kb[c] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rk, vlane, base + c * 1024u, 0));
    };
    auto load_v = [&](int v, bf16x8_t (&Vb)[2 * DB]) {
        const uint32_t base = half_base(v) + uint32_t(v & 1) * 2 * 1024u;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                Vb[2 * db + cc] = as_bf16x8(
                    __builtin_amdgcn_raw_buffer_load_b128(rv, vlane, base + (4 * db + cc) * 1024u, 0));
    };

    f32x16_t O[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db][0] = O[db][1] = f32x16_t{};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    const float c2 = a.scale_log2e;
    const int n_half = n_key_tiles * HPU;  // always even

    // One 32-key half: S = K.Q^T, online softmax, O += V.P; then refill the
    // buffers with half v + 2 (two halves in flight while this one computes).
    // The body is straight-line on purpose: halves with no real key are masked
    // rather than skipped, and the last two refills re-read a valid half, so
    // the ring registers never merge values from different control paths.
    auto step = [&](int v, bf16x8_t (&Kb)[NC], bf16x8_t (&Vb)[2 * DB]) {
        const int real = min(32, bl_s[half_tile(v)] - 32 * (v % HPU));
        const int next = v + 2 < n_half ? v + 2 : v;

        // S^T[qb]: rows = keys 8i + 4*half + j of this half (acc 4i + j), col = query.
        // The Q fragments are re-read from LDS each half: the empty asm makes the
        // lane index opaque so the reads are not hoisted into 64 live VGPRs.
        int ql = lane;
        asm volatile("" : "+v"(ql));
        f32x16_t S[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Kb[c], q_lds[qb][c][ql], acc, 0, 0, 0);
            S[qb] = acc;
        }
        load_k(next, Kb);
        // Padding keys (partial tiles only: a wave-uniform branch) never score.
        if (__builtin_expect(real < 32, 0)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (8 * i + 4 * half + j >= real) {
                        S[0][4 * i + j] = -INFINITY;
                        S[1][4 * i + j] = -INFINITY;
                    }
        }

        // Online softmax per query column, rescaling lazily: the running max m
        // only moves (and O, l are rescaled) when some row's new max exceeds it
        // by more than kLazy in log2 units, so p <= 2^kLazy stays safe in fp32
        // and bf16 while most halves skip the rescale entirely.
        float mx[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float t = S[qb][0];
#pragma unroll
            for (int e = 1; e < 16; ++e) t = fmaxf(t, S[qb][e]);
            mx[qb] = fmaxf(t, __shfl_xor(t, 32));
        }
        const bool grow = (mx[0] * c2 > m[0] * c2 + kLazy) || (mx[1] * c2 > m[1] * c2 + kLazy);
        if (__ballot(grow) != 0) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float m_new = fmaxf(m[qb], mx[qb]);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m[qb] - m_new) * c2);
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) O[db][qb][e] *= alpha;
                m[qb] = m_new;
            }
        }
        bf16x8_t Pf[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float moff = m[qb] == -INFINITY ? 0.f : -m[qb] * c2;
            float rs = 0.f;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][8 * cc + e], c2, moff));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][8 * cc + e + 1], c2, moff));
                    const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
                    rs = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, rs, false);
                    w[e / 2] = __builtin_bit_cast(uint32_t, pp);
                }
                // 16-key chunk cc of this half = acc elements 8cc .. 8cc + 7
                Pf[qb][cc] = as_bf16x8(w);
            }
            rs += __shfl_xor(rs, 32);
            l[qb] += rs;
        }

        // O^T[db][qb] += V^T[db] . P^T[qb] over the half's two 16-key chunks.
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                f32x16_t acc = O[db][qb];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Vb[2 * db + cc], Pf[qb][cc], acc, 0, 0, 0);
                O[db][qb] = acc;
            }
        load_v(next, Vb);
    };

    bf16x8_t K0[NC], V0[2 * DB], K1[NC], V1[2 * DB];
    load_k(0, K0);
    load_v(0, V0);
    load_k(1, K1);
    load_v(1, V1);
    for (int v = 0; v < n_half; v += 2) {
        step(v, K0, V0);
        step(v + 1, K1, V1);
    }

    // ---- epilogue: out = bf16(O_fine + g * O_coarse[tile]), natural token order.
    // O^T[db][qb] acc 4i + j <-> d = 32db + 8i + 4*half + j, query column l32.
    const float *oc = a.o_coarse + (size_t(h) * a.n_t + tile) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if (tok[qb] < 0) continue;
        const float inv = 1.0f / l[qb];
        const size_t base = (size_t(tok[qb]) * a.H + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * half;
                const float4 ocv = *reinterpret_cast<const float4 *>(oc + d0);
                const uint2 graw = *reinterpret_cast<const uint2 *>(a.gate + base + d0);
                const float g0 = __uint_as_float(graw.x << 16), g1 = __uint_as_float(graw.x & 0xffff0000u);
                const float g2 = __uint_as_float(graw.y << 16), g3 = __uint_as_float(graw.y & 0xffff0000u);
                const float r0 = O[db][qb][4 * i + 0] * inv + g0 * ocv.x;
                const float r1 = O[db][qb][4 * i + 1] * inv + g1 * ocv.y;
                const float r2 = O[db][qb][4 * i + 2] * inv + g2 * ocv.z;
                const float r3 = O[db][qb][4 * i + 3] * inv + g3 * ocv.w;
                const bf16x2_t w0 = {(__bf16)r0, (__bf16)r1}, w1 = {(__bf16)r2, (__bf16)r3};
                uint2 w;
                w.x = *reinterpret_cast<const uint32_t *>(&w0);
                w.y = *reinterpret_cast<const uint32_t *>(&w1);
                *reinterpret_cast<uint2 *>(a.out + base + d0) = w;
            }
    }
}

template <int D, int B>
void launch_fine(const FineArgs &a, hipStream_t st)
{
    const int items = a.H * a.n_t * (B / 64);
    hipLaunchKernelGGL((fine_attn_kernel<D, B>), dim3(items), dim3(64), 0, st, a);
}

}  // namespace
}  // namespace vsa

using namespace vsa;

extern "C" int vsa_sparse_attn_fwd(const vsa_plan_info *info, const int32_t *row_src_dev,
                                   const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                   int32_t k, float scale, const void *q, const void *workspace,
                                   size_t workspace_bytes, const int32_t *keep_idx_dev,
                                   const float *o_coarse_dev, const void *gate, void *out,
                                   void *stream)
{
    clear_error();
    if (int st = check_info(info)) return st;
    if (heads <= 0) return fail(VSA_ERR_ARG, "heads = %d", heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "head_dim = %d; supported: 64, 128", head_dim);
    if (k < 0 || k > info->n_video_tiles)
        return fail(VSA_ERR_ARG, "k = %d outside [0, %d]", k, info->n_video_tiles);
    if (info->n_prefix_tiles == 0 && k == 0 && info->n_video_tiles > 0)
        return fail(VSA_ERR_ARG, "empty key set: no prefix tiles and k = 0");
    if (!row_src_dev || !block_len_dev || !q || !workspace || !o_coarse_dev || !gate || !out)
        return fail(VSA_ERR_ARG, "null device pointer");
    if (k > 0 && !keep_idx_dev) return fail(VSA_ERR_ARG, "keep_idx is null with k = %d", k);
    if (!std::isfinite(scale)) return fail(VSA_ERR_ARG, "scale is not finite");
    vsa_ws_layout L;
    compute_layout(*info, heads, head_dim, &L);
    if (workspace_bytes < L.total_bytes)
        return fail(VSA_ERR_ARG, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(VSA_ERR_ARG, "workspace must be 256-byte aligned");
    if (int st = check_device()) return st;

    const char *ws = static_cast<const char *>(workspace);
    FineArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.kt = reinterpret_cast<const uint16_t *>(ws + L.k_tiled);
    a.vt = reinterpret_cast<const uint16_t *>(ws + L.v_tiled);
    a.row_src = row_src_dev;
    a.block_len = block_len_dev;
    a.keep = keep_idx_dev;
    a.o_coarse = o_coarse_dev;
    a.gate = static_cast<const uint16_t *>(gate);
    a.out = static_cast<uint16_t *>(out);
    a.H = heads;
    a.P = info->n_prefix_tiles;
    a.n_v = info->n_video_tiles;
    a.n_t = info->n_tiles;
    a.k = k;
    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(float(head_dim));
    a.scale_log2e = sc * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int B = info->tile_rows;
    if (head_dim == 128) {
        if (B == 64) launch_fine<128, 64>(a, st);
        else launch_fine<128, 128>(a, st);
    } else {
        if (B == 64) launch_fine<64, 64>(a, st);
        else launch_fine<64, 128>(a, st);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return VSA_OK;
}
