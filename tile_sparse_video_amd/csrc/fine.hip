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

template <int D>
struct Frags {
    bf16x8_t x[2][D / 16];  // [32-row block][16-wide reduction chunk]
};

__device__ __forceinline__ bf16x8_t load_frag(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8_t *>(p);
}

template <int D, int B>
__global__ __launch_bounds__(64) void fine_attn_kernel(FineArgs a)
{
    constexpr int SUB = B / 64;   // 64-row blocks per tile
    constexpr int NC = D / 16;    // reduction chunks of S = K.Q^T
    constexpr int DB = D / 32;    // 32-row blocks of O^T (over d)
    constexpr int FR = D / 8;     // fragments per 64-row block
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
    const int32_t *keep_row = dense ? nullptr : a.keep + (size_t(h) * a.n_v + (tile - a.P)) * a.k;

    // ---- query fragments (B operand of S^T = K . Q^T): lane -> query 32qb + l32,
    // reduction slot e of chunk c -> d = 16c + 8*half + e.
    int tok[2];
    Frags<D> Qf;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        tok[qb] = a.row_src[size_t(tile) * B + 64 * qsub + 32 * qb + l32];
        const uint16_t *qrow = a.q + (size_t(tok[qb] < 0 ? 0 : tok[qb]) * a.H + h) * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8_t v = load_frag(qrow + 16 * c);
            if (tok[qb] < 0) v = bf16x8_t{};
            Qf.x[qb][c] = v;
        }
    }

    // Kept tiles come from the coarse stage; clamping only guards against a
    // foreign keep list addressing outside the workspace.
    auto key_tile = [&](int n) -> int {
        return (dense || n < a.P) ? n : min(max(keep_row[n - a.P], 0), a.n_t - 1);
    };
    auto frag_base = [&](const uint16_t *t, int kt_id, int s) -> const uint16_t * {
        return t + ((size_t(h) * a.n_t + kt_id) * SUB + s) * FR * 512 + lane * 8;
    };

    f32x16_t O[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db][0] = O[db][1] = f32x16_t{};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    const float c2 = a.scale_log2e;

    const int n_units = n_key_tiles * SUB;
    int cur_tile = key_tile(0);
    Frags<D> Kf;
    {
        const uint16_t *kp = frag_base(a.kt, cur_tile, 0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < NC; ++c) Kf.x[kb][c] = load_frag(kp + (kb * NC + c) * 512);
    }

    for (int u = 0; u < n_units; ++u) {
        const int s = u % SUB;
        const int real = min(64, a.block_len[cur_tile] - 64 * s);

        // V of this unit: A operand of O^T += V^T . P^T (fragment f = db*4 + c).
        bf16x8_t Vf[DB][4];
        {
            const uint16_t *vp = frag_base(a.vt, cur_tile, s);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int c = 0; c < 4; ++c) Vf[db][c] = load_frag(vp + (db * 4 + c) * 512);
        }

        // S^T[kb][qb]: rows = keys 32kb + 8i + 4*half + j (acc 4i + j), col = query.
        f32x16_t S[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                f32x16_t acc = f32x16_t{};
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Kf.x[kb][c], Qf.x[qb][c], acc, 0, 0, 0);
                S[kb][qb] = acc;
            }

        // Prefetch the next unit's K while the softmax and P.V of this one run.
        const int nu = u + 1;
        int next_tile = cur_tile;
        if (nu < n_units) {
            next_tile = (nu % SUB == 0) ? key_tile(nu / SUB) : cur_tile;
            const uint16_t *kp = frag_base(a.kt, next_tile, nu % SUB);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int c = 0; c < NC; ++c) Kf.x[kb][c] = load_frag(kp + (kb * NC + c) * 512);
        }

        // Mask padding keys, then the online softmax per query column.
        if (real < 64) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (32 * kb + 8 * i + 4 * half + j >= real) {
                            S[kb][0][4 * i + j] = -INFINITY;
                            S[kb][1][4 * i + j] = -INFINITY;
                        }
        }
        bf16x8_t Pf[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[kb][qb][e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m[qb], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2f((m[qb] - m_use) * c2);
            const float moff = -m_use * c2;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                uint16_t pb[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = exp2f(__builtin_fmaf(S[kb][qb][e], c2, moff));
                    rs += p;
                    pb[e] = f32_to_bf16(p);
                }
                // chunk c = 2kb + half16 holds acc elements 8*half16 .. 8*half16 + 7
                Pf[qb][2 * kb + 0] = *reinterpret_cast<bf16x8_t *>(&pb[0]);
                Pf[qb][2 * kb + 1] = *reinterpret_cast<bf16x8_t *>(&pb[8]);
            }
            rs += __shfl_xor(rs, 32);
            l[qb] = l[qb] * alpha + rs;
            m[qb] = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) O[db][qb][e] *= alpha;
        }

        // O^T[db][qb] += V^T[db] . P^T[qb] over the four 16-key chunks.
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                f32x16_t acc = O[db][qb];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Vf[db][c], Pf[qb][c], acc, 0, 0, 0);
                O[db][qb] = acc;
            }
        cur_tile = next_tile;
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
                uint2 w;
                w.x = uint32_t(f32_to_bf16(r0)) | (uint32_t(f32_to_bf16(r1)) << 16);
                w.y = uint32_t(f32_to_bf16(r2)) | (uint32_t(f32_to_bf16(r3)) << 16);
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
