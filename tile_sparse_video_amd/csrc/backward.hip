// Backward pass of gated, tile-sparse video attention on gfx950: the gradient
// of the layer with respect to Q, K, V and the gate, with the keep sets held
// fixed (a top-k selection has no gradient).
//
// Method: SnackOnAI analysis of ComfyUI-Ref2VA-VSA, "References" (VSA trains
// end to end with its sparse kernel) and "The Code, Annotated", snippet two
// (the forward being differentiated: sink prefix tiles, block_len masking,
// scale = D^-1/2); the Veda news item's reference_sparsity input for the
// explicit-list variant.
//
// Forward, per head, for a real token t of tile i:
//   O_fine[t] = sum_{u in keys(i)} softmax_u(scale q_t.k_u) v_u
//   O_c[i]    = sum_j softmax_j(scale qm_i.km_j) vm_j   (tile means, all tiles)
//   out[t]    = O_fine[t] + g[t] * O_c[i]
// Kernels, in launch order:
//   frag_gather  -- V / Q / dO in the row-fragment layout, K / Q / dO in the
//                   column-fragment layout (the two MFMA operand layouts of
//                   the forward's K and V copies), tile order, padding zero;
//   bwd_prep     -- dg = dout * O_c and dO_c[i] = sum_{t in i} dout * g;
//   coarse_bwd   -- the tile-level attention's gradient to the tile means
//                   (fp32, rows then columns);
//   tlist        -- for every key tile, the ascending list of query tiles
//                   whose key list holds it (the transpose of the keep sets);
//   dq           -- query-major: the fine forward again (log-sum-exp, O_fine
//                   and the softmax-gradient row term D_t = dout . O_fine),
//                   then dQ = scale dS K over the tile's key list, plus the
//                   mean's share dqm / n;
//   dkdv         -- key-major over the transposed lists: dV = P^T dO,
//                   dK = scale dS^T Q, plus dkm / n and dvm / n.
// S, dP, dV and dK run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
// P and dS rounded to bf16 as the forward rounds P.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "device.h"

namespace vsa {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource word 3, 32-bit data (gfx9 family)

// Packs fp32 values a[8 cc .. 8 cc + 7] into the bf16 B operand of one 16-row
// chunk (the accumulator-to-operand order the forward uses for P).
__device__ __forceinline__ bf16x8_t pack8(const f32x16_t &a, int cc)
{
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2_t pp = {(__bf16)a[8 * cc + e], (__bf16)a[8 * cc + e + 1]};
        w[e / 2] = __builtin_bit_cast(uint32_t, pp);
    }
    return as_bf16x8(w);
}

// ----------------------------------------------------------- frag_gather --
//
// One block per (tile, group of 256/D heads). ROWS = 1: row layout, fragment
// f = kb*(D/16) + c holds row 32kb + l32, d = 16c + 8*half + e. ROWS = 0:
// column layout, fragment f = db*4 + c holds d = 32db + l32, rows 16c +
// {4h..4h+3, 8+4h..8+4h+3}. The same two layouts the coarse stage writes for K
// and V. ROWS = 2: both, from one staged tile (dst: row layout, dst_col:
// column layout), for the tensors the backward needs in both (Q, dO).
template <int D, int B, int ROWS>
__global__ __launch_bounds__(256) void frag_gather_kernel(const uint16_t *__restrict__ X,
                                                         const int32_t *__restrict__ row_src,
                                                         const int32_t *__restrict__ block_len,
                                                         int H, int n_t, uint16_t *__restrict__ dst,
                                                         uint16_t *__restrict__ dst_col = nullptr)
{
    constexpr int HPB = 256 / D, ROW = HPB * D + 8, CH = HPB * D / 8, FR = D / 8, SUB = B / 64;
    __shared__ __attribute__((aligned(16))) uint16_t lds[B * ROW];
    __shared__ int32_t toks[B];
    const int tile = blockIdx.x, h0 = blockIdx.y * HPB, tid = threadIdx.x;
    const int nh = min(HPB, H - h0), n = block_len[tile];
    if (tid < B) toks[tid] = row_src[size_t(tile) * B + tid];
    __syncthreads();
    for (int idx = tid; idx < B * CH; idx += 256) {
        const int r = idx / CH, c = idx % CH;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < n && c / (D / 8) < nh)
            val = *reinterpret_cast<const uint4 *>(X + (size_t(toks[r]) * H + h0) * D + c * 8);
        *reinterpret_cast<uint4 *>(&lds[r * ROW + c * 8]) = val;
    }
    __syncthreads();
    const int total = nh * SUB * FR * kWave;
    for (int idx = tid; idx < total; idx += 256) {
        const int lane = idx % kWave, f = (idx / kWave) % FR;
        const int sub = (idx / (kWave * FR)) % SUB, hl = idx / (kWave * FR * SUB);
        const int half = lane / 32, l32 = lane % 32;
        const size_t frag = ((size_t(h0 + hl) * n_t + tile) * SUB + sub) * FR + f;
        if (ROWS != 0) {
            const int kb = f / (D / 16), c = f % (D / 16);
            const uint16_t *src = &lds[(64 * sub + 32 * kb + l32) * ROW + hl * D + 16 * c + 8 * half];
            *reinterpret_cast<uint4 *>(dst + frag * 512 + lane * 8) = *reinterpret_cast<const uint4 *>(src);
        }
        if (ROWS != 1) {
            uint16_t e8[8];
            const int db = f / 4, c = f % 4;
            const int col = hl * D + 32 * db + l32, r0 = 64 * sub + 16 * c + 4 * half;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                e8[e] = lds[(r0 + e) * ROW + col];
                e8[4 + e] = lds[(r0 + 8 + e) * ROW + col];
            }
            *reinterpret_cast<uint4 *>((ROWS == 2 ? dst_col : dst) + frag * 512 + lane * 8) =
                *reinterpret_cast<uint4 *>(e8);
        }
    }
}

// -------------------------------------------------------------- bwd_prep --
//
// One block (4 waves) per (tile, head); wave w takes the tile's real rows
// w, w+4, ...; lane owns d = lane + 64p. Writes dg (fp32, natural order) and
// dO_c[i] = sum over the tile's rows of dout * g.
template <int D, int B>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t *__restrict__ dout,
                                                      const uint16_t *__restrict__ gate,
                                                      const float *__restrict__ o_coarse,
                                                      const int32_t *__restrict__ row_src,
                                                      const int32_t *__restrict__ block_len, int H,
                                                      int n_t, float *__restrict__ dgate,
                                                      float *__restrict__ doc)
{
    constexpr int PL = D / kWave;
    __shared__ float red[4][D];
    const int tile = blockIdx.x, h = blockIdx.y;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int n = block_len[tile];
    float oc[PL], acc[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        oc[p] = o_coarse[(size_t(h) * n_t + tile) * D + lane + kWave * p];
        acc[p] = 0.f;
    }
    for (int r = w; r < n; r += 4) {
        const int t = row_src[size_t(tile) * B + r];
        const size_t base = (size_t(t) * H + h) * D;
#pragma unroll
        for (int p = 0; p < PL; ++p) {
            const int d = lane + kWave * p;
            const float go = bf16_to_f32(dout[base + d]);
            const float g = bf16_to_f32(gate[base + d]);
            dgate[base + d] = go * oc[p];
            acc[p] += go * g;
        }
    }
#pragma unroll
    for (int p = 0; p < PL; ++p) red[w][lane + kWave * p] = acc[p];
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += 256)
        doc[(size_t(h) * n_t + tile) * D + d] = red[0][d] + red[1][d] + red[2][d] + red[3][d];
}

// ------------------------------------------------------------ coarse_bwd --
//
// Tile-level attention gradient in fp32 on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32), laid out as the forward's coarse attention: a
// workgroup of 4 waves covers 128 tiles of a head, blocks of 32 partner tiles
// are staged in LDS, and each MFMA contracts the reduction index of lane half
// h with the one of the other half. Softmax in the log2 domain: with
// c = scale log2 e, P_ij = exp2(c qm_i.km_j - lse_i), lse_i = log2 sum_j
// exp2(c qm_i.km_j) (stored in lsec in that domain).
//
// Rows: lane = query tile i. Pass 1: lse_i (online max and sum). Pass 2:
// dZ_ij = scale P_ij (dO_c[i].vm_j - Dc_i) and dqm_i = sum_j dZ_ij km_j; also
// Dc_i = dO_c[i] . O_c[i].
template <int D>
__global__ __launch_bounds__(256) void coarse_bwd_rows_kernel(const float *__restrict__ qm,
                                                             const float *__restrict__ km,
                                                             const float *__restrict__ vm,
                                                             const float *__restrict__ o_coarse,
                                                             const float *__restrict__ doc, int n_t,
                                                             float scale, float *__restrict__ lsec,
                                                             float *__restrict__ dcc,
                                                             float *__restrict__ dqm)
{
    constexpr int KB = 32, ROW = D + 1, HD = D / 2, DB = D / 32;
    __shared__ float ks[KB * ROW];
    __shared__ float vs[KB * ROW];
    const int h = blockIdx.y, wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int l32 = lane & 31, half = lane >> 5;
    const size_t hb = size_t(h) * n_t * D;
    const int qi = blockIdx.x * 128 + wave * 32 + l32;
    const bool qlive = qi < n_t;
    const float c2 = scale * 1.4426950408889634f;

    // B operands: lane -> query column l32, reduction slots d = HD half + m.
    float qv[HD], gv[HD];
    float dc = 0.f;
#pragma unroll
    for (int m = 0; m < HD; ++m) {
        const size_t at = hb + size_t(qlive ? qi : 0) * D + HD * half + m;
        qv[m] = qlive ? qm[at] : 0.f;
        gv[m] = qlive ? doc[at] : 0.f;
        dc += gv[m] * (qlive ? o_coarse[at] : 0.f);
    }
    dc += __shfl_xor(dc, 32);

    auto stage = [&](int j0, bool with_v) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < KB * D; idx += 256) {
            const int r = idx / D, c = idx % D;
            const bool live = j0 + r < n_t;
            ks[r * ROW + c] = live ? km[hb + size_t(j0 + r) * D + c] : 0.f;
            if (with_v) vs[r * ROW + c] = live ? vm[hb + size_t(j0 + r) * D + c] : 0.f;
        }
        __syncthreads();
    };
    // S^T = K . Q^T: rows = keys 8i + 4 half + j of the block (acc 4i + j), column = query.
    auto scores = [&](int j0) {
        f32x16_t S = f32x16_t{};
#pragma unroll
        for (int m = 0; m < HD; ++m)
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[l32 * ROW + HD * half + m], qv[m], S, 0, 0, 0);
        if (j0 + KB > n_t) {  // key tiles past the end never score
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j0 + 8 * i + 4 * half + j >= n_t) S[4 * i + j] = -INFINITY;
        }
        return S;
    };

    // pass 1: lse (log2 domain) over all key tiles
    float mrun = -INFINITY, lrun = 0.f;
    for (int j0 = 0; j0 < n_t; j0 += KB) {
        stage(j0, false);
        const f32x16_t S = scores(j0);
        float mx = S[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(mrun, mx);  // finite: every block has a real key tile
        float rs = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) rs += __builtin_amdgcn_exp2f((S[e] - m_new) * c2);
        rs += __shfl_xor(rs, 32);
        lrun = lrun * __builtin_amdgcn_exp2f((mrun - m_new) * c2) + rs;
        mrun = m_new;
    }
    const float lse = mrun * c2 + __log2f(lrun);

    // pass 2: dQm^T += K^T dZ^T; product m pairs keys 8(m/4) + 4 half + m%4,
    // the S accumulator elements the lane holds.
    f32x16_t G[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) G[db] = f32x16_t{};
    for (int j0 = 0; j0 < n_t; j0 += KB) {
        stage(j0, true);
        const f32x16_t S = scores(j0);
        f32x16_t dP = f32x16_t{};
#pragma unroll
        for (int m = 0; m < HD; ++m)
            dP = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[l32 * ROW + HD * half + m], gv[m], dP, 0, 0, 0);
        float dz[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c2, -lse));
            dz[e] = p * (dP[e] - dc) * scale;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            f32x16_t acc = G[db];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int key = 8 * (m / 4) + 4 * half + (m % 4);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[key * ROW + 32 * db + l32], dz[m], acc, 0, 0, 0);
            }
            G[db] = acc;
        }
    }
    if (!qlive) return;
    // G[db] element 4i + j <-> d = 32db + 8i + 4 half + j, query column l32.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            *reinterpret_cast<float4 *>(dqm + hb + size_t(qi) * D + d0) =
                make_float4(G[db][4 * i], G[db][4 * i + 1], G[db][4 * i + 2], G[db][4 * i + 3]);
        }
    if (half == 0) {
        lsec[size_t(h) * n_t + qi] = lse;
        dcc[size_t(h) * n_t + qi] = dc;
    }
}

// Columns: lane = key tile j; blocks of 32 query tiles (means of Q and dO_c,
// their lse and Dc) are staged in LDS. S = Q K^T and dP = dO_c V^T with rows =
// queries 8i + 4 half + j (acc 4i + j); then dKm^T += Q^T dZ and dVm^T +=
// dO_c^T P, product m pairing queries 8(m/4) + 4 half + m%4.
template <int D>
__global__ __launch_bounds__(256) void coarse_bwd_cols_kernel(const float *__restrict__ qm,
                                                             const float *__restrict__ km,
                                                             const float *__restrict__ vm,
                                                             const float *__restrict__ doc,
                                                             const float *__restrict__ lsec,
                                                             const float *__restrict__ dcc, int n_t,
                                                             float scale, float *__restrict__ dkm,
                                                             float *__restrict__ dvm)
{
    constexpr int QB = 32, ROW = D + 1, HD = D / 2, DB = D / 32;
    __shared__ float qs[QB * ROW];
    __shared__ float gs[QB * ROW];
    __shared__ float ls[QB], cs[QB];
    const int h = blockIdx.y, wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int l32 = lane & 31, half = lane >> 5;
    const size_t hb = size_t(h) * n_t * D;
    const int kj = blockIdx.x * 128 + wave * 32 + l32;
    const bool klive = kj < n_t;
    const float c2 = scale * 1.4426950408889634f;

    float kv[HD], vv[HD];
#pragma unroll
    for (int m = 0; m < HD; ++m) {
        const size_t at = hb + size_t(klive ? kj : 0) * D + HD * half + m;
        kv[m] = klive ? km[at] : 0.f;
        vv[m] = klive ? vm[at] : 0.f;
    }
    f32x16_t GK[DB], GV[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) GK[db] = GV[db] = f32x16_t{};
    for (int i0 = 0; i0 < n_t; i0 += QB) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < QB * D; idx += 256) {
            const int r = idx / D, c = idx % D;
            const bool live = i0 + r < n_t;
            qs[r * ROW + c] = live ? qm[hb + size_t(i0 + r) * D + c] : 0.f;
            gs[r * ROW + c] = live ? doc[hb + size_t(i0 + r) * D + c] : 0.f;
        }
        if (threadIdx.x < QB) {
            const bool live = i0 + int(threadIdx.x) < n_t;
            ls[threadIdx.x] = live ? lsec[size_t(h) * n_t + i0 + threadIdx.x] : INFINITY;  // P = 0
            cs[threadIdx.x] = live ? dcc[size_t(h) * n_t + i0 + threadIdx.x] : 0.f;
        }
        __syncthreads();
        f32x16_t S = f32x16_t{}, dP = f32x16_t{};
#pragma unroll
        for (int m = 0; m < HD; ++m) {
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[l32 * ROW + HD * half + m], kv[m], S, 0, 0, 0);
            dP = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[l32 * ROW + HD * half + m], vv[m], dP, 0, 0, 0);
        }
        float p[16], dz[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int qr = 8 * (e / 4) + 4 * half + (e % 4);
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c2, -ls[qr]));
            dz[e] = p[e] * (dP[e] - cs[qr]) * scale;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            f32x16_t ak = GK[db], av = GV[db];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int qr = 8 * (m / 4) + 4 * half + (m % 4);
                ak = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[qr * ROW + 32 * db + l32], dz[m], ak, 0, 0, 0);
                av = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[qr * ROW + 32 * db + l32], p[m], av, 0, 0, 0);
            }
            GK[db] = ak;
            GV[db] = av;
        }
    }
    if (!klive) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            *reinterpret_cast<float4 *>(dkm + hb + size_t(kj) * D + d0) =
                make_float4(GK[db][4 * i], GK[db][4 * i + 1], GK[db][4 * i + 2], GK[db][4 * i + 3]);
            *reinterpret_cast<float4 *>(dvm + hb + size_t(kj) * D + d0) =
                make_float4(GV[db][4 * i], GV[db][4 * i + 1], GV[db][4 * i + 2], GV[db][4 * i + 3]);
        }
}

// ----------------------------------------------------------------- tlist --
//
// The transpose of the key lists, in two passes over a bit matrix
// bits[h][i][w] (W = ceil(n_t / 32) words per query tile i; bit j set when
// query tile i's key list holds key tile j):
//   tbits_kernel: one wavefront per (query tile, head) sets the bits of its
//     list in an LDS row (prefix key tiles and dense rows as whole-word masks,
//     kept tiles with LDS atomic ors, which commute) and stores the row;
//   tlist_kernel: one wavefront per (key tile j, head) reads bit j of every
//     row (independent loads, eight per lane in flight) and compacts the query
//     tiles that have it with ballots, in ascending order.
// Both are exact and deterministic; no step depends on the order of atomics.

// Bits [32 w, 32 w + 32) of the range [0, n) as a word.
__device__ __forceinline__ uint32_t range_word(int w, int n)
{
    const int lo = 32 * w, left = n - lo;
    return left <= 0 ? 0u : left >= 32 ? 0xffffffffu : (1u << left) - 1u;
}

__global__ __launch_bounds__(256) void tbits_kernel(const int32_t *__restrict__ keep, int ref, int P,
                                                    int n_v, int n_t, int k, int list_len, int W,
                                                    uint32_t *__restrict__ bits)
{
    extern __shared__ uint32_t rows[];  // [4][W]
    const int h = blockIdx.y, wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int i = blockIdx.x * 4 + wave;
    const bool live = i < n_t;  // no early return: the block's barriers stay uniform
    uint32_t *row = rows + wave * W;
    const bool dense = !ref && i < P;
    // Initial words: a dense row holds every key tile; a default-mode row the
    // prefix key tiles [0, P); a reference-mode row starts empty.
    for (int w = lane; w < W; w += kWave) row[w] = !live ? 0u : dense ? range_word(w, n_t) : ref ? 0u : range_word(w, P);
    __syncthreads();
    if (live && !dense) {
        const int len = ref ? list_len : k;
        const int32_t *src = ref ? keep + (size_t(h) * n_t + i) * list_len : keep + (size_t(h) * n_v + (i - P)) * k;
        for (int s = lane; s < len; s += kWave) {
            const int j = min(max(src[s], 0), n_t - 1);
            atomicOr(&row[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    if (live)
        for (int w = lane; w < W; w += kWave) bits[(size_t(h) * n_t + i) * W + w] = row[w];
}

constexpr int kTlistBatch = 8;  // rows read per lane before their ballots

__global__ __launch_bounds__(256) void tlist_kernel(const uint32_t *__restrict__ bits, int n_t, int W,
                                                    int32_t *__restrict__ tlist,
                                                    int32_t *__restrict__ tcount)
{
    const int h = blockIdx.y;
    const int j = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (j >= n_t) return;
    const uint32_t *col = bits + size_t(h) * n_t * W + (j >> 5);
    const uint32_t bit = 1u << (j & 31);
    int32_t *dst = tlist + (size_t(h) * n_t + j) * n_t;
    int count = 0;
    for (int i0 = 0; i0 < n_t; i0 += kWave * kTlistBatch) {
        uint32_t word[kTlistBatch];
#pragma unroll
        for (int u = 0; u < kTlistBatch; ++u)  // clamped rows: every load issued, none behind a branch
            word[u] = col[size_t(min(i0 + kWave * u + lane, n_t - 1)) * W];
#pragma unroll
        for (int u = 0; u < kTlistBatch; ++u) {
            const int i = i0 + kWave * u + lane;
            const bool has = i < n_t && (word[u] & bit) != 0u;
            const uint64_t m = __ballot(has);
            if (has) dst[count + __popcll(m & lanes_below(lane))] = i;
            count += __popcll(m);
        }
    }
    if (lane == 0) tcount[size_t(h) * n_t + j] = count;
}

struct BwdArgs {
    const uint16_t *q, *dout;       // natural [S][H][D]
    const uint16_t *kt, *vt;        // forward workspace: K row fragments, V column fragments
    const uint16_t *vrow, *kcol;    // V row fragments, K column fragments
    const uint16_t *qcol, *docol;   // Q and dO column fragments
    const uint16_t *qrow, *dorow;   // Q and dO row fragments
    const uint16_t *kn, *vn;        // natural K and V
    const int32_t *row_src, *block_len, *keep;
    const int32_t *tlist, *tcount;
    const float *dt;                // [H][S_pad] D_t, written by the dq kernel (dt_out)
    float *dt_out;
    float *lse;                     // [H][S_pad], log2 domain (+inf on padding rows)
    const float *dqm, *dkm, *dvm;   // [H][n_t][D]
    float *dq, *dk, *dv;            // natural [S][H][D]
    float *part_dq;                 // split dq: [items][8][D/32][2][4][64][4] fp32
    float *part_dkv;                // split dk/dv: [H][n_t][8][B/32][2][D/32][4][64][4] fp32
    int H, P, n_v, n_t, k, ref, list_len;
    float scale, scale_log2e;
};

// -------------------------------------------------------------------- dq --
//
// One wavefront per (head, 64 query rows), as the forward: Q and dO fragments
// staged in LDS, K / V / K^T fragments streamed as 1 KB coalesced buffer loads
// per 32-key half. Pass 1 forms S^T = K Q^T and the per-query log-sum-exp
// (written for the key-major kernel); pass 2 forms S^T, P^T, dP^T = V dO^T,
// dS^T = P^T (dP^T - D) and dQ^T += K^T dS^T.
template <int D, int B, bool SPLIT>
__global__ __launch_bounds__(64, 1) void dq_kernel(BwdArgs a)
{
    constexpr int SUB = B / 64, NC = D / 16, DB = D / 32, FR = D / 8, HPU = 2 * SUB;
    constexpr int kListCap = 896;
    const int lane = threadIdx.x, l32 = lane & 31, half = lane >> 5;
    const int per_head = a.n_t * SUB;
    // Split: 8 chunks by key tile id mod 8, chunk = block % 8 so that chunk c
    // runs on XCD c (as the forward); the log-sum-exp and D_t come from the
    // statistics pass and each chunk writes a partial dQ.
    const int item = SPLIT ? int(blockIdx.x / 8) : int(blockIdx.x);
    const int chunk = SPLIT ? int(blockIdx.x % 8) : 0;
    const int h = item / per_head, r = item % per_head;
    const int tile = r / SUB, qsub = r % SUB;
    const bool dense = !a.ref && tile < a.P;
    const int n_list = a.ref ? a.list_len : dense ? a.n_t : a.P + a.k;
    const size_t S_pad = size_t(a.n_t) * B;

    __shared__ __attribute__((aligned(16))) bf16x8_t q_lds[2][NC][kWave];
    __shared__ __attribute__((aligned(16))) bf16x8_t o_lds[2][NC][kWave];
    __shared__ uint32_t list_lds[kListCap];
    int tok[2];
    float dq_row[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) tok[qb] = a.row_src[tile * B + 64 * qsub + 32 * qb + l32];
    // The block's 64 Q and dO rows, D / 8 lanes per row (16 bytes each, so a
    // load covers whole rows), stored to their fragment slots: piece p of row
    // r is chunk p / 2, slot half p % 2, column r % 32 of block r / 32.
    {
        constexpr int PPR = D / 8, RPI = kWave / PPR, NG = 64 / RPI;
        const int pr = lane / PPR, pp = lane % PPR;
        size_t rbase[NG];
        bool real[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int tk = a.row_src[tile * B + 64 * qsub + RPI * g + pr];
            real[g] = tk >= 0;
            rbase[g] = (size_t(tk < 0 ? 0 : tk) * a.H + h) * D + 8 * pp;
        }
#pragma unroll
        for (int src = 0; src < 2; ++src) {
            const uint16_t *p = src == 0 ? a.q : a.dout;
            bf16x8_t v[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(p + rbase[g]);
                v[g] = real[g] ? x : bf16x8_t{};
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int r = RPI * g + pr;
                (src == 0 ? q_lds : o_lds)[r >> 5][pp >> 1][(pp & 1) * 32 + (r & 31)] = v[g];
            }
        }
    }
    const int32_t *keep_row = a.ref ? a.keep + (size_t(h) * a.n_t + tile) * a.list_len
                              : dense ? a.keep
                                      : a.keep + (size_t(h) * a.n_v + (tile - a.P)) * a.k;
    auto tile_at = [&](int n) -> int {
        if (a.ref) return min(max(keep_row[n], 0), a.n_t - 1);
        return (dense || n < a.P) ? n : min(max(keep_row[n - a.P], 0), a.n_t - 1);
    };
    const uint32_t head_bytes = uint32_t(a.n_t) * B * D * 2;
    const size_t head_elems = size_t(h) * a.n_t * B * D;
    auto rsrc = [&](const uint16_t *p) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)(p + head_elems), (short)0, head_bytes, kRsrcWord3);
    };
    const __amdgpu_buffer_rsrc_t rk = rsrc(a.kt), rvr = rsrc(a.vrow), rkc = rsrc(a.kcol);
    const int vlane = lane * 16;
    const float c2 = a.scale_log2e;

    // Walks the key list in segments staged in LDS. Per 32-key half v:
    // fetch(v, entry, regs) issues its operand loads, body(v, entry, regs)
    // uses them; the next half's loads are in flight while the current half
    // is computed (two register sets; a segment always has an even number of
    // halves).
    auto walk = [&](auto &&fetch, auto &&body, auto &regA, auto &regB) {
        int scan = 0;
        while (true) {
            int count = 0;
            while (scan < n_list) {
                const int n = scan + lane;
                int t = n < n_list ? tile_at(n) : -1;
                if (SPLIT && t % 8 != chunk) t = -1;
                const uint64_t mask = __ballot(t >= 0);
                const int take = __popcll(mask);
                if (count + take > kListCap) break;
                if (t >= 0) list_lds[count + __popcll(mask & lanes_below(lane))] = uint32_t(t) | uint32_t(a.block_len[t] - 1) << 25;
                count += take;
                scan += kWave;
            }
            __syncthreads();
            const int n_half = count * HPU;
            auto ent = [&](int v) { return __builtin_amdgcn_readfirstlane(list_lds[v / HPU]); };
            // Halves v (even) and v + 1 lie in one tile, so they share an entry;
            // the next tile's entry is read before this pair's products, so no
            // half waits on an LDS round trip.
            uint32_t e = n_half > 0 ? ent(0) : 0u;
            if (n_half > 0) fetch(0, e, regA);
            for (int v = 0; v < n_half; v += 2) {
                fetch(v + 1, e, regB);
                const uint32_t e2 = ent(min(v + 2, n_half - 1));
                body(v, e, regA);
                if (v + 2 < n_half) fetch(v + 2, e2, regA);
                body(v + 1, e, regB);
                e = e2;
            }
            if (scan >= n_list) break;
            __syncthreads();
        }
    };
    auto half_base = [&](int v, uint32_t ent) -> uint32_t {
        return ((ent & 0x1ffffffu) * SUB + uint32_t((v % HPU) >> 1)) * FR * 1024u;
    };
    // A . B^T with A = 32 key rows (fragments in registers) and B = the Q (or dO)
    // rows of query block qb from LDS; the lane index is made opaque so the LDS
    // operands are re-read rather than hoisted into VGPRs.
    auto s_block = [&](int qb, const u32x4_t (&Kb)[NC], bool use_do) {
        int ql = lane;
        asm volatile("" : "+v"(ql));
        f32x16_t S = f32x16_t{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bf16x8_t bq = use_do ? o_lds[qb][c][ql] : q_lds[qb][c][ql];
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Kb[c]), bq, S, 0, 0, 0);
        }
        return S;
    };
    auto mask_pad = [&](f32x16_t &S, int real) {
        if (__builtin_expect(real < 32, 0)) {  // partial tiles only: a wave-uniform branch
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (8 * i + 4 * half + j >= real) S[4 * i + j] = -INFINITY;
        }
    };

    // ---- pass 1: the fine forward again -- running max, sum and O^T = V^T P^T
    // -- giving the log-sum-exp (log2 domain) and D_t = dout . O_fine, both
    // written for the key-major kernel.
    const __amdgpu_buffer_rsrc_t rv = rsrc(a.vt);
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    f32x16_t O[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db][0] = O[db][1] = f32x16_t{};
    struct Regs1 {
        u32x4_t Kb[NC], Vc[2 * DB];
    };
    auto fetch1 = [&](int v, uint32_t ent, Regs1 &g) {
        const uint32_t hb = half_base(v, ent);
        const uint32_t base = hb + uint32_t(v & 1) * NC * 1024u;
        const uint32_t cbase = hb + uint32_t(v & 1) * 2 * 1024u;
#pragma unroll
        for (int c = 0; c < NC; ++c) g.Kb[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, vlane, base + c * 1024u, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                g.Vc[2 * db + cc] = __builtin_amdgcn_raw_buffer_load_b128(rv, vlane, cbase + (4 * db + cc) * 1024u, 0);
    };
    auto body1 = [&](int v, uint32_t ent, const Regs1 &g) {
        const int real = min(32, int(ent >> 25) + 1 - 32 * (v % HPU));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x16_t S = s_block(qb, g.Kb, false);
            mask_pad(S, real);
            float mx = S[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m[qb], mx);
            if (mn > m[qb]) {  // per query column; VALU only
                const float alpha = m[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m[qb] - mn) * c2);
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) O[db][qb][e] *= alpha;
                m[qb] = mn;
            }
            // A column with no real key yet (all -inf) takes P = 0, not NaN.
            const float mref = mn == -INFINITY ? 0.f : mn;
            f32x16_t Pm;
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                Pm[e] = __builtin_amdgcn_exp2f((S[e] - mref) * c2);
                s += Pm[e];
            }
            l[qb] += s + __shfl_xor(s, 32);
            const bf16x8_t p0 = pack8(Pm, 0), p1 = pack8(Pm, 1);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(g.Vc[2 * db]), p0, O[db][qb], 0, 0, 0);
                O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(g.Vc[2 * db + 1]), p1, O[db][qb], 0, 0, 0);
            }
        }
    };
    float lse[2];
    if (SPLIT) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const size_t row = size_t(h) * S_pad + tile * B + 64 * qsub + 32 * qb + l32;
            lse[qb] = a.lse[row];
            dq_row[qb] = a.dt[row];
        }
    } else {
        Regs1 ga, gb;
        walk(fetch1, body1, ga, gb);
    }
#pragma unroll
    for (int qb = 0; qb < 2 && !SPLIT; ++qb) {
        const size_t row = size_t(h) * S_pad + tile * B + 64 * qsub + 32 * qb + l32;
        // D_t = sum_d dout[d] O_fine[d]; O^T acc 4i + j <-> d = 32db + 8i + 4 half + j.
        float part = 0.f;
        if (tok[qb] >= 0) {
            const uint16_t *go = a.dout + (size_t(tok[qb]) * a.H + h) * D;
            const float inv = 1.0f / l[qb];
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint2 raw = *reinterpret_cast<const uint2 *>(go + 32 * db + 8 * i + 4 * half);
                    part += __uint_as_float(raw.x << 16) * O[db][qb][4 * i] * inv;
                    part += __uint_as_float(raw.x & 0xffff0000u) * O[db][qb][4 * i + 1] * inv;
                    part += __uint_as_float(raw.y << 16) * O[db][qb][4 * i + 2] * inv;
                    part += __uint_as_float(raw.y & 0xffff0000u) * O[db][qb][4 * i + 3] * inv;
                }
        }
        dq_row[qb] = part + __shfl_xor(part, 32);
        lse[qb] = tok[qb] < 0 ? INFINITY : m[qb] * c2 + __log2f(l[qb]);
        if (half == 0) {
            a.lse[row] = lse[qb];
            a.dt_out[row] = dq_row[qb];
        }
    }

    // ---- pass 2: dQ^T = K^T dS^T
    f32x16_t G[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) G[db][0] = G[db][1] = f32x16_t{};
    struct Regs2 {
        u32x4_t Kb[NC], Vr[NC], Kc[2 * DB];
    };
    auto fetch2 = [&](int v, uint32_t ent, Regs2 &g) {
        const uint32_t hb = half_base(v, ent);
        const uint32_t kbase = hb + uint32_t(v & 1) * NC * 1024u;
        const uint32_t cbase = hb + uint32_t(v & 1) * 2 * 1024u;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            g.Kb[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, vlane, kbase + c * 1024u, 0);
            g.Vr[c] = __builtin_amdgcn_raw_buffer_load_b128(rvr, vlane, kbase + c * 1024u, 0);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                g.Kc[2 * db + cc] = __builtin_amdgcn_raw_buffer_load_b128(rkc, vlane, cbase + (4 * db + cc) * 1024u, 0);
    };
    auto body2 = [&](int v, uint32_t ent, const Regs2 &g) {
        const int real = min(32, int(ent >> 25) + 1 - 32 * (v % HPU));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x16_t S = s_block(qb, g.Kb, false);
            mask_pad(S, real);
            const f32x16_t dP = s_block(qb, g.Vr, true);
            f32x16_t dS;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c2, -lse[qb]));
                dS[e] = p * (dP[e] - dq_row[qb]);
            }
            const bf16x8_t d0 = pack8(dS, 0), d1 = pack8(dS, 1);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                G[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(g.Kc[2 * db]), d0, G[db][qb], 0, 0, 0);
                G[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(g.Kc[2 * db + 1]), d1, G[db][qb], 0, 0, 0);
            }
        }
    };
    {
        Regs2 ga, gb;
        walk(fetch2, body2, ga, gb);
    }

    if (SPLIT) {
        // partial dQ^T of this chunk, fp32: [item][8][DB][2][4][64][4], register
        // group q4 of every lane in one lane-contiguous 1 KB run. Only the merge
        // reads it: non-temporal stores keep it from displacing reused K/V in L2.
        float *pd = a.part_dq + (size_t(item) * 8 + chunk) * (DB * 2 * kWave * 16);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float4 *dst = reinterpret_cast<float4 *>(pd + (db * 2 + qb) * kWave * 16);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    __builtin_nontemporal_store(f32x4_t{G[db][qb][4 * q4], G[db][qb][4 * q4 + 1], G[db][qb][4 * q4 + 2],
                                                        G[db][qb][4 * q4 + 3]},
                                                reinterpret_cast<f32x4_t *>(dst + q4 * kWave + lane));
            }
        return;
    }
    // ---- epilogue: dq = scale dQ_fine + dqm / n (fp32, natural order)
    const float inv_n = 1.0f / float(a.block_len[tile]);
    const float *gm = a.dqm + (size_t(h) * a.n_t + tile) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if (tok[qb] < 0) continue;
        float *dst = a.dq + (size_t(tok[qb]) * a.H + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * half;
                const float4 mm = *reinterpret_cast<const float4 *>(gm + d0);
                float4 o;
                o.x = a.scale * G[db][qb][4 * i] + mm.x * inv_n;
                o.y = a.scale * G[db][qb][4 * i + 1] + mm.y * inv_n;
                o.z = a.scale * G[db][qb][4 * i + 2] + mm.z * inv_n;
                o.w = a.scale * G[db][qb][4 * i + 3] + mm.w * inv_n;
                *reinterpret_cast<float4 *>(dst + d0) = o;
            }
    }
}

// Sums the 8 chunk partials of one item (in chunk order) and writes
// dq = scale dQ_fine + dqm / n. One wavefront per (item, 32-row half qb,
// 32-column block db), lanes as the dq kernel: its 32 partial loads are
// independent and in flight together, and the many small waves hide the
// latency of one another.
template <int D, int B>
__global__ __launch_bounds__(256) void dq_merge_kernel(BwdArgs a, int n_items)
{
    constexpr int SUB = B / 64, DB = D / 32;
    const int lane = threadIdx.x % kWave, half = lane >> 5, l32 = lane & 31;
    const int wid = blockIdx.x * 4 + threadIdx.x / kWave;
    if (wid >= n_items * 2 * DB) return;
    // Tile-major numbering (the heads of one 64-row block side by side): the
    // fp32 dq rows that neighbouring waves write lie in the same token records.
    const int grp = wid / (2 * DB), qb = (wid / DB) % 2, db = wid % DB;
    const int h = grp % a.H, r = grp / a.H;
    const int item = h * (a.n_t * SUB) + r;
    const int tile = r / SUB, qsub = r % SUB;
    const int tok = a.row_src[size_t(tile) * B + 64 * qsub + 32 * qb + l32];
    const float inv_n = 1.0f / float(a.block_len[tile]);
    const float *gm = a.dqm + (size_t(h) * a.n_t + tile) * D + 32 * db + 4 * half;
    float acc[16] = {};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float4 *src = reinterpret_cast<const float4 *>(
            a.part_dq + (size_t(item) * 8 + c) * (DB * 2 * kWave * 16) + (db * 2 + qb) * kWave * 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(src + q4 * kWave + lane));
            acc[4 * q4] += v[0];
            acc[4 * q4 + 1] += v[1];
            acc[4 * q4 + 2] += v[2];
            acc[4 * q4 + 3] += v[3];
        }
    }
    float4 mm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mm[i] = *reinterpret_cast<const float4 *>(gm + 8 * i);
    if (tok < 0) return;
    float *dst = a.dq + (size_t(tok) * a.H + h) * D + 32 * db + 4 * half;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4 *>(dst + 8 * i) =
            make_float4(a.scale * acc[4 * i] + mm[i].x * inv_n, a.scale * acc[4 * i + 1] + mm[i].y * inv_n,
                        a.scale * acc[4 * i + 2] + mm[i].z * inv_n, a.scale * acc[4 * i + 3] + mm[i].w * inv_n);
}

// ------------------------------------------------------------------ dkdv --
//
// Heads too small to split (the split ones use dkdv_ring_kernel below).
// One wavefront per (head, key tile, 32 key rows), the key tile's waves in one
// workgroup. The wave holds its keys' K^T and V^T operand fragments (natural rows) and the dK^T, dV^T
// accumulators (lane = key column), and walks the query tiles of the key
// tile's transposed list, 32 query rows (one "block") at a time:
//   S = Q K^T, P = exp2(S c2 - lse), dP = dO V^T, dS = P (dP - D),
//   dV^T += dO^T P, dK^T += Q^T dS.
// Every operand is a coalesced 1 KB fragment of the tile-ordered copies; the
// row-layout operands and row statistics of the next block are fetched while
// the current one is computed (two register sets, the loop unrolled by two).
// The dK^T, dV^T accumulators stay in AGPRs for the whole walk.
template <int D, int B>
__global__ __launch_bounds__(B * 2, 1) void dkdv_kernel(BwdArgs a)
{
    constexpr int SUB = B / 64, NC = D / 16, DB = D / 32, FR = D / 8;
    // One workgroup per (head, key tile): wave kb owns key rows 32kb..32kb+31.
    // The waves walk the same query list in step, so the second wave's
    // fragment reads are served by the CU's L1.
    const int lane = threadIdx.x % kWave, l32 = lane & 31, half = lane >> 5;
    const int kb = threadIdx.x / kWave;
    const int ht = int(blockIdx.x);
    const int h = ht / a.n_t, tile = ht % a.n_t;
    const size_t S_pad = size_t(a.n_t) * B;

    // Own keys as B operands: lane -> key 32kb + l32 of the tile, slots d = 16c + 8 half + e.
    const int krow = tile * B + 32 * kb + l32;
    const int ktok = a.row_src[krow];
    bf16x8_t Kt[NC], Vt[NC];
    {
        const size_t base = (size_t(ktok < 0 ? 0 : ktok) * a.H + h) * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            Kt[c] = *reinterpret_cast<const bf16x8_t *>(a.kn + base + 16 * c);
            Vt[c] = *reinterpret_cast<const bf16x8_t *>(a.vn + base + 16 * c);
            if (ktok < 0) Kt[c] = Vt[c] = bf16x8_t{};
        }
    }
    f32x16_t GK[DB], GV[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) GK[db] = GV[db] = f32x16_t{};
    const float c2 = a.scale_log2e;

    const int cnt = a.tcount[size_t(h) * a.n_t + tile];
    const int32_t *lst = a.tlist + (size_t(h) * a.n_t + tile) * a.n_t;
    const int n_blocks = cnt * SUB * 2;  // 32-row query blocks (even)

    // Operands of block b: query tile lst[b / (2 SUB)], 64-row block (b / 2) % SUB, half b % 2.
    struct RowOps {
        u32x4_t Qr[NC], Or[NC];
        float4 L4[4], D4[4];
    };
    // Operands are read through buffer resources based at the head's region:
    // the lane's 16-byte slot is the VGPR offset and the block's fragment
    // offset is uniform (SGPR), so no address arithmetic runs per load.
    const uint32_t frag_bytes = uint32_t(S_pad) * D * 2;
    const size_t head_elems = size_t(h) * S_pad * D;
    auto rsrc = [&](const uint16_t *p) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)(p + head_elems), (short)0, frag_bytes, kRsrcWord3);
    };
    const __amdgpu_buffer_rsrc_t rqr = rsrc(a.qrow), ror = rsrc(a.dorow), rqc = rsrc(a.qcol), roc = rsrc(a.docol);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.lse + size_t(h) * S_pad), (short)0, uint32_t(S_pad) * 4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.dt + size_t(h) * S_pad), (short)0, uint32_t(S_pad) * 4, kRsrcWord3);
    const int vlane = lane * 16, vrow = (4 * half) * 4;
    auto fbyte = [&](int b) -> uint32_t {
        const int qt = __builtin_amdgcn_readfirstlane(lst[b / (2 * SUB)]);
        return uint32_t(qt * SUB + (b / 2) % SUB) * FR * 1024u;
    };
    auto fetch = [&](int b, RowOps &o) {
        const int qt = __builtin_amdgcn_readfirstlane(lst[b / (2 * SUB)]);
        const int sub = (b / 2) % SUB, qb = b % 2;
        const uint32_t fb = uint32_t(qt * SUB + sub) * FR * 1024u;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            o.Qr[c] = __builtin_amdgcn_raw_buffer_load_b128(rqr, vlane, fb + (qb * NC + c) * 1024u, 0);
            o.Or[c] = __builtin_amdgcn_raw_buffer_load_b128(ror, vlane, fb + (qb * NC + c) * 1024u, 0);
        }
        const uint32_t r0 = uint32_t(qt * B + 64 * sub + 32 * qb) * 4u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_t l = __builtin_amdgcn_raw_buffer_load_b128(rl, vrow, r0 + 32u * i, 0);
            const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(rd, vrow, r0 + 32u * i, 0);
            o.L4[i] = make_float4(__uint_as_float(l[0]), __uint_as_float(l[1]), __uint_as_float(l[2]), __uint_as_float(l[3]));
            o.D4[i] = make_float4(__uint_as_float(d[0]), __uint_as_float(d[1]), __uint_as_float(d[2]), __uint_as_float(d[3]));
        }
    };
    auto compute = [&](int b, const RowOps &o) {
        const uint32_t fb = fbyte(b);
        const int qb = b % 2;
        f32x16_t S = f32x16_t{}, dP = f32x16_t{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(o.Qr[c]), Kt[c], S, 0, 0, 0);
            dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(o.Or[c]), Vt[c], dP, 0, 0, 0);
        }
        u32x4_t Oc[2 * DB], Qc[2 * DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint32_t off = fb + (4 * db + 2 * qb + cc) * 1024u;
                Oc[2 * db + cc] = __builtin_amdgcn_raw_buffer_load_b128(roc, vlane, off, 0);
                Qc[2 * db + cc] = __builtin_amdgcn_raw_buffer_load_b128(rqc, vlane, off, 0);
            }
        f32x16_t Pm, dS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lv[4] = {o.L4[i].x, o.L4[i].y, o.L4[i].z, o.L4[i].w};
            const float dv[4] = {o.D4[i].x, o.D4[i].y, o.D4[i].z, o.D4[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p = __builtin_amdgcn_exp2f(S[4 * i + j] * c2 - lv[j]);
                Pm[4 * i + j] = p;
                dS[4 * i + j] = p * (dP[4 * i + j] - dv[j]);
            }
        }
        const bf16x8_t p0 = pack8(Pm, 0), p1 = pack8(Pm, 1);
        const bf16x8_t s0 = pack8(dS, 0), s1 = pack8(dS, 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            GV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Oc[2 * db]), p0, GV[db], 0, 0, 0);
            GV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Oc[2 * db + 1]), p1, GV[db], 0, 0, 0);
            GK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Qc[2 * db]), s0, GK[db], 0, 0, 0);
            GK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Qc[2 * db + 1]), s1, GK[db], 0, 0, 0);
        }
    };
    if (n_blocks > 0) {
        RowOps A, Bo;
        fetch(0, A);
        for (int b = 0; b < n_blocks; b += 2) {
            fetch(b + 1, Bo);
            compute(b, A);
            if (b + 2 < n_blocks) fetch(b + 2, A);
            compute(b + 1, Bo);
        }
    }
    if (ktok < 0) return;
    // dk = scale dK_fine + dkm / n, dv = dV_fine + dvm / n; acc 4i + j <-> d = 32db + 8i + 4 half + j.
    const float inv_n = 1.0f / float(a.block_len[tile]);
    const float *gk = a.dkm + (size_t(h) * a.n_t + tile) * D;
    const float *gv = a.dvm + (size_t(h) * a.n_t + tile) * D;
    float *dk = a.dk + (size_t(ktok) * a.H + h) * D;
    float *dv = a.dv + (size_t(ktok) * a.H + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            const float4 mk = *reinterpret_cast<const float4 *>(gk + d0);
            const float4 mv = *reinterpret_cast<const float4 *>(gv + d0);
            float4 ok, ov;
            ok.x = a.scale * GK[db][4 * i] + mk.x * inv_n;
            ok.y = a.scale * GK[db][4 * i + 1] + mk.y * inv_n;
            ok.z = a.scale * GK[db][4 * i + 2] + mk.z * inv_n;
            ok.w = a.scale * GK[db][4 * i + 3] + mk.w * inv_n;
            ov.x = GV[db][4 * i] + mv.x * inv_n;
            ov.y = GV[db][4 * i + 1] + mv.y * inv_n;
            ov.z = GV[db][4 * i + 2] + mv.z * inv_n;
            ov.w = GV[db][4 * i + 3] + mv.w * inv_n;
            *reinterpret_cast<float4 *>(dk + d0) = ok;
            *reinterpret_cast<float4 *>(dv + d0) = ov;
        }
}

// ------------------------------------------------------------- dkdv ring --
//
// The dK/dV pass for split heads with the query-side operands shared through
// LDS. A workgroup (one key tile, one chunk of its transposed list; wave kb
// owns key rows 32kb..32kb+31 with their K^T, V^T in registers and dK^T, dV^T
// in AGPRs) walks 32-row query blocks through a ring of NBUF LDS stages. A
// stage holds the block's Q and dO row fragments (1 KB each, the tile-ordered
// copies) and the lse and D_t of its rows; the column-layout operands of the
// dV and dK products are read from the same row fragments with the LDS
// transpose read (ds_read_b64_tr_b16), so Q and dO cross from L2 once. The
// waves fill a stage together with buffer-to-LDS loads (each wave a fixed
// share of the fragments plus one row-statistics load: wave 0 the lse,
// wave 1 the D_t, further waves a spare copy), so a fragment crosses from L2
// once per workgroup and never occupies VGPRs in flight; a stage is refilled
// NBUF - 1 blocks ahead of its use. Every wave issues the same number of
// loads per block (past the end of the list it reloads the last block into
// the free stage), so one wait on its own load counter, then a plain barrier,
// makes the whole stage visible; a second barrier after the reads frees the
// stage. Nothing else in the loop issues vector-memory loads, so the load
// counter counts exactly the ring's loads.
template <int D, int B>
struct RingCfg {
    static constexpr int NC = D / 16, DB = D / 32, KB = B / 32;
    static constexpr int FRAGS = 2 * NC;                // Qr, Or fragments per block
    static constexpr int LPW = FRAGS / KB;              // fragment loads per wave per block
    static constexpr int NBUF = 4;                      // stages (B = 64: two workgroups per CU)
    // Fragments are staged 1024 + 64 bytes apart: the column reads of the dV and dK
    // products take two neighbouring fragments at once, and the padding puts them
    // on different LDS banks.
    static constexpr int FST = 1024 + 64;
    static constexpr int STAGE = FRAGS * FST + KB * 256;  // + 64 lse, 64 D_t (+ spare areas)
    static constexpr int LIST = 4096;                   // uint16 query-tile ids of the chunk
    static constexpr size_t LDS = size_t(NBUF) * STAGE + LIST * 2;
};

// s_waitcnt immediate (gfx9 encoding) waiting until at most n vector-memory
// loads are outstanding, with the export and LDS counters left alone.
#define VSA_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int D, int B>
__global__ __launch_bounds__(B * 2, 1) void dkdv_ring_kernel(BwdArgs a)
{
    using C = RingCfg<D, B>;
    constexpr int SUB = B / 64, NC = C::NC, DB = C::DB, FR = D / 8, KB = C::KB;
    constexpr int NBUF = C::NBUF, LPW = C::LPW, STAGE = C::STAGE;
    extern __shared__ __attribute__((aligned(16))) char ring_lds[];
    uint16_t *flist = reinterpret_cast<uint16_t *>(ring_lds + size_t(NBUF) * STAGE);
    const int lane = threadIdx.x % kWave, l32 = lane & 31, half = lane >> 5;
    const int kb = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
    const int ht = blockIdx.x / 8, chunk = blockIdx.x % 8;
    const int h = ht / a.n_t, tile = ht % a.n_t;
    const size_t S_pad = size_t(a.n_t) * B;

    // Own keys as B operands: lane -> key 32kb + l32 of the tile, slots d = 16c + 8 half + e.
    const int ktok = a.row_src[tile * B + 32 * kb + l32];
    bf16x8_t Kt[NC], Vt[NC];
    {
        const size_t base = (size_t(ktok < 0 ? 0 : ktok) * a.H + h) * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            Kt[c] = *reinterpret_cast<const bf16x8_t *>(a.kn + base + 16 * c);
            Vt[c] = *reinterpret_cast<const bf16x8_t *>(a.vn + base + 16 * c);
            if (ktok < 0) Kt[c] = Vt[c] = bf16x8_t{};
        }
    }
    f32x16_t GK[DB], GV[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) GK[db] = GV[db] = f32x16_t{};
    const float c2 = a.scale_log2e;

    // This chunk's query tiles (id % 8 == chunk), compacted in order by wave 0.
    if (kb == 0) {
        const int cnt_all = a.tcount[size_t(h) * a.n_t + tile];
        const int32_t *lst = a.tlist + (size_t(h) * a.n_t + tile) * a.n_t;
        int n = 0;
        for (int x0 = 0; x0 < cnt_all; x0 += kWave) {
            const int x = x0 + lane;
            const int qt = x < cnt_all ? lst[x] : -1;
            const bool m = qt >= 0 && qt % 8 == chunk;
            const uint64_t bal = __ballot(m);
            if (m) flist[n + __popcll(bal & lanes_below(lane))] = uint16_t(qt);
            n += __popcll(bal);
        }
        if (lane == 0) flist[C::LIST - 1] = uint16_t(n);
    }
    __syncthreads();  // also orders the key loads above before the ring's load counting
    const int n_blocks = int(flist[C::LIST - 1]) * SUB * 2;

    const uint32_t frag_bytes = uint32_t(S_pad) * D * 2;
    const size_t head_elems = size_t(h) * S_pad * D;
    auto rsrc = [&](const uint16_t *p) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)(p + head_elems), (short)0, frag_bytes, kRsrcWord3);
    };
    const __amdgpu_buffer_rsrc_t rqr = rsrc(a.qrow), ror = rsrc(a.dorow);
    // Transposed reads. A row fragment chunk c holds, at byte 16 l + 2 e, the
    // block's row l % 32, d = 16c + 8 (l / 32) + e. ds_read_b64_tr_b16 gives
    // lane i of each 16-lane group the element i % 4 of the 8-byte segments
    // that lanes i / 4 + 4k (k < 4) address. For the column fragment (db, cc)
    // (lane L: d = 32 db + L % 32, rows 16 cc + 4 (L / 32) + {0..3} and
    // + 8 + {0..3}) lane j of group g therefore addresses row
    // 16 cc + 4 (g / 2) + j / 4 at d = 32 db + 16 (g % 2) + 4 (j % 4); the second
    // read adds 8 rows. The per-lane part of that address is fixed.
    const int tg = lane >> 4, ti = lane & 15;
    const int t_d0 = 16 * (tg & 1) + 4 * (ti & 3);                    // d - 32 db
    const uint32_t t_base = uint32_t(((t_d0 >> 4) * C::FST) +                 // chunk 2 db + g % 2
                                     ((4 * (tg >> 1) + (ti >> 2)) + 32 * ((t_d0 >> 3) & 1)) * 16 +
                                     2 * (t_d0 & 7));
    // Row statistics: wave 0 reads lse, the others D_t (only wave 1's copy is used).
    const uint64_t stat_base = reinterpret_cast<uint64_t>((kb == 0 ? a.lse : a.dt) + size_t(h) * S_pad);
    const uint64_t stat_uni = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(stat_base)))) |
                              uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(stat_base >> 32)))) << 32;
    const __amdgpu_buffer_rsrc_t rstat = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(stat_uni), (short)0, uint32_t(S_pad) * 4, kRsrcWord3);

    // Issue this wave's loads of block b into stage `slot`: fragments
    // j = kb*LPW + t (Qr c for j < NC, then Or c) and 64 row
    // statistics from the block's first row (lanes 0-31 are the block's rows;
    // rows past the head's end read as zero).
    auto issue = [&](int b, int slot) {
        const int qt = __builtin_amdgcn_readfirstlane(int(flist[b / (2 * SUB)]));
        const int sub = (b / 2) % SUB, qb = b % 2;
        const uint32_t fb = uint32_t(qt * SUB + sub) * FR * 1024u;
        char *stage = ring_lds + slot * STAGE;
#pragma unroll
        for (int t = 0; t < LPW; ++t) {
            const int j = kb * LPW + t;
            const __amdgpu_buffer_rsrc_t r = j < NC ? rqr : ror;
            const uint32_t f = qb * NC + (j < NC ? j : j - NC);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void *)(stage + j * C::FST), 16, lane * 16, fb + f * 1024u, 0, 0);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rstat, (__attribute__((address_space(3))) void *)(stage + C::FRAGS * C::FST + kb * 256), 4, lane * 4,
            uint32_t(qt * B + 64 * sub + 32 * qb) * 4u, 0, 0);
    };
    // Phase 1 of block b: S = Q K^T and dP = dO V^T from the row fragments.
    auto phase1 = [&](int b, f32x16_t &S, f32x16_t &dP) {
        const char *stage = ring_lds + (b % NBUF) * STAGE;
        auto frag = [&](int j) { return *reinterpret_cast<const bf16x8_t *>(stage + j * C::FST + lane * 16); };
        S = f32x16_t{};
        dP = f32x16_t{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(c), Kt[c], S, 0, 0, 0);
            dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(NC + c), Vt[c], dP, 0, 0, 0);
        }
    };
    // One step of the loop: block b's softmax terms, each pair of elements
    // placed between two of block b + 1's S and dP products (those only read
    // the next stage, so the matrix core and the vector unit work side by
    // side), then block b's dV and dK products. Past the list's end the S and dP
    // products of the reloaded last block run and are never used.
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    auto step = [&](int b, const f32x16_t &S, const f32x16_t &dP, f32x16_t &Sn, f32x16_t &dPn) {
        const int nb = b + NBUF - 1;
        issue(nb < n_blocks ? nb : n_blocks - 1, nb % NBUF);  // into the stage freed by block b - 1
        __builtin_amdgcn_s_waitcnt(VSA_VMCNT((NBUF - 2) * (LPW + 1)));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();     // every wave's part of stage (b + 1) % NBUF has landed
        asm volatile("" ::: "memory");
        const char *stage = ring_lds + (b % NBUF) * STAGE;
        const char *nstage = ring_lds + ((b + 1) % NBUF) * STAGE;
        // Row statistics of block b: lse at rows 8i + 4 half + j (i, j < 4) and
        // D_t 256 bytes further, read in one asm block that also waits for them
        // (the compiler sees no LDS load it would order after a wait for every
        // buffer-to-LDS load in flight). Early-clobber outputs: the address is
        // still read after the first result is written.
        f32x4_t L[4], Dv[4];
        const uint32_t st_addr = uint32_t(reinterpret_cast<uintptr_t>(stage)) + C::FRAGS * C::FST + 16 * half;
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:32\n\t"
            "ds_read_b128 %2, %8 offset:64\n\t"
            "ds_read_b128 %3, %8 offset:96\n\t"
            "ds_read_b128 %4, %8 offset:256\n\t"
            "ds_read_b128 %5, %8 offset:288\n\t"
            "ds_read_b128 %6, %8 offset:320\n\t"
            "ds_read_b128 %7, %8 offset:352\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(L[0]), "=&v"(L[1]), "=&v"(L[2]), "=&v"(L[3]), "=&v"(Dv[0]), "=&v"(Dv[1]), "=&v"(Dv[2]),
              "=&v"(Dv[3])
            : "v"(st_addr)
            : "memory");
        auto nfrag = [&](int j) { return *reinterpret_cast<const bf16x8_t *>(nstage + j * C::FST + lane * 16); };
        bf16x8_t FQ[NC], FO[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            FQ[c] = nfrag(c);
            FO[c] = nfrag(NC + c);
        }
        // Column fragment (db, cc) of the Q (first = 0) or dO (first = NC) chunks.
        auto col = [&](int first, int db, int cc) -> bf16x8_t {
            typedef short s16x4_t __attribute__((ext_vector_type(4)));
            const char *p = stage + first * C::FST + t_base + 2 * C::FST * db + 256 * cc;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t *)(p));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t *)(p + 128));
            const u32x4_t w = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
            return as_bf16x8(w);
        };
        Sn = f32x16_t{};
        dPn = f32x16_t{};
        f32x16_t Pm, dS;
        bf16x8_t CO[DB][2], CQ[DB][2];  // block b's column fragments of dO and Q
        constexpr int EPG = 16 / NC;  // softmax elements per pair of products
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int u = 0; u < EPG; ++u) {
                const int e = EPG * c + u, i = e / 4, j = e % 4;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c2, -L[i][j]));
                Pm[e] = p;
                dS[e] = p * (dP[e] - Dv[i][j]);
            }
            Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FQ[c], Kt[c], Sn, 0, 0, 0);
            dPn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FO[c], Vt[c], dPn, 0, 0, 0);
#pragma unroll
            for (int q = c * 2 * DB / NC; q < (c + 1) * 2 * DB / NC; ++q) {
                CO[q / 2][q % 2] = col(NC, q / 2, q % 2);
                CQ[q / 2][q % 2] = col(0, q / 2, q % 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const bf16x8_t p0 = pack8(Pm, 0), p1 = pack8(Pm, 1);
        const bf16x8_t s0 = pack8(dS, 0), s1 = pack8(dS, 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            GV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CO[db][0], p0, GV[db], 0, 0, 0);
            GV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CO[db][1], p1, GV[db], 0, 0, 0);
            GK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CQ[db][0], s0, GK[db], 0, 0, 0);
            GK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CQ[db][1], s1, GK[db], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS reads of stage b % NBUF done (lgkmcnt 0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();     // stage b % NBUF may be refilled
        asm volatile("" ::: "memory");
    };
    if (n_blocks > 0) {
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) issue(min(b, n_blocks - 1), b);
        __builtin_amdgcn_s_waitcnt(VSA_VMCNT((NBUF - 2) * (LPW + 1)));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();     // stage 0 has landed
        asm volatile("" ::: "memory");
        f32x16_t Sa, dPa, Sb, dPb;
        phase1(0, Sa, dPa);
        for (int b = 0; b < n_blocks; b += 2) {  // n_blocks is even
            step(b, Sa, dPa, Sb, dPb);
            step(b + 1, Sb, dPb, Sa, dPa);
        }
    }
    // partial dK^T, dV^T, fp32: [H][n_t][8][KB][2][DB][4][64][4], register group
    // q4 of every lane in one lane-contiguous 1 KB run.
    float *pd = a.part_dkv + ((size_t(ht) * 8 + chunk) * KB + kb) * (2 * DB * kWave * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        float4 *dk4 = reinterpret_cast<float4 *>(pd + db * kWave * 16);
        float4 *dv4 = reinterpret_cast<float4 *>(pd + (DB + db) * kWave * 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            __builtin_nontemporal_store(f32x4_t{GK[db][4 * q4], GK[db][4 * q4 + 1], GK[db][4 * q4 + 2], GK[db][4 * q4 + 3]},
                                        reinterpret_cast<f32x4_t *>(dk4 + q4 * kWave + lane));
            __builtin_nontemporal_store(f32x4_t{GV[db][4 * q4], GV[db][4 * q4 + 1], GV[db][4 * q4 + 2], GV[db][4 * q4 + 3]},
                                        reinterpret_cast<f32x4_t *>(dv4 + q4 * kWave + lane));
        }
    }
}
#undef VSA_VMCNT

// Raises the dynamic-LDS limit of the ring kernel once per process.
template <int D, int B>
int ring_lds_attr()
{
    static const int status =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&dkdv_ring_kernel<D, B>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(RingCfg<D, B>::LDS)) == hipSuccess
            ? int(VSA_OK)
            : int(VSA_ERR_DEVICE);
    return status;
}

// Sums the 8 chunk partials of one (head, key tile, 32 key rows) in chunk
// order and writes dk = scale dK + dkm / n, dv = dV + dvm / n for real keys.
// One wavefront per (unit, dk or dv, 32-column block db): its 32 partial
// loads are independent and in flight together.
template <int D, int B>
__global__ __launch_bounds__(256) void dkdv_merge_kernel(BwdArgs a, int n_units)
{
    constexpr int DB = D / 32, KB = B / 32;
    const int lane = threadIdx.x % kWave, half = lane >> 5, l32 = lane & 31;
    const int wid = blockIdx.x * 4 + threadIdx.x / kWave;
    if (wid >= n_units * 2 * DB) return;
    // Tile-major numbering, as in dq_merge_kernel.
    const int grp = wid / (2 * DB), kv = (wid / DB) % 2, db = wid % DB;
    const int h = grp % a.H, rest = grp / a.H;
    const int tile = rest / KB, kb = rest % KB;
    const int ht = h * a.n_t + tile;
    const int ktok = a.row_src[size_t(tile) * B + 32 * kb + l32];
    const float inv_n = 1.0f / float(a.block_len[tile]);
    const float *gm = (kv == 0 ? a.dkm : a.dvm) + (size_t(h) * a.n_t + tile) * D + 32 * db + 4 * half;
    float acc[16] = {};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float4 *src = reinterpret_cast<const float4 *>(
            a.part_dkv + ((size_t(ht) * 8 + c) * KB + kb) * (2 * DB * kWave * 16) + (kv * DB + db) * kWave * 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(src + q4 * kWave + lane));
            acc[4 * q4] += v[0];
            acc[4 * q4 + 1] += v[1];
            acc[4 * q4 + 2] += v[2];
            acc[4 * q4 + 3] += v[3];
        }
    }
    float4 mm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mm[i] = *reinterpret_cast<const float4 *>(gm + 8 * i);
    if (ktok < 0) return;
    const float sc = kv == 0 ? a.scale : 1.0f;
    float *dst = (kv == 0 ? a.dk : a.dv) + (size_t(ktok) * a.H + h) * D + 32 * db + 4 * half;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4 *>(dst + 8 * i) =
            make_float4(sc * acc[4 * i] + mm[i].x * inv_n, sc * acc[4 * i + 1] + mm[i].y * inv_n,
                        sc * acc[4 * i + 2] + mm[i].z * inv_n, sc * acc[4 * i + 3] + mm[i].w * inv_n);
}

}  // namespace
}  // namespace vsa

namespace vsa {

// The dK/dV pass splits its query lists into 8 XCD-affine chunks when the
// heads are large (as the forward) and the fp32 partials stay within 64 GiB.
bool dkdv_split(const vsa_plan_info &info, int heads, int head_dim, int chunks)
{
    const double bytes = double(heads) * info.n_tiles * 8 * (info.tile_rows / 32) * 2 * 32 * head_dim * 4;
    return chunks > 1 && info.n_tiles <= 4095 && bytes <= 64.0 * (1 << 30);
}

void compute_bwd_layout(const vsa_plan_info &info, int heads, int head_dim, int chunks, vsa_bwd_layout *L)
{
    const size_t H = size_t(heads), D = size_t(head_dim), n_t = size_t(info.n_tiles);
    const size_t S_pad = size_t(info.rows_padded);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    L->vrow = take(H * S_pad * D * 2);
    L->kcol = take(H * S_pad * D * 2);
    L->qcol = take(H * S_pad * D * 2);
    L->docol = take(H * S_pad * D * 2);
    L->qrow = take(H * S_pad * D * 2);
    L->dorow = take(H * S_pad * D * 2);
    L->lse = take(H * S_pad * 4);
    L->dt = take(H * S_pad * 4);
    L->doc = take(H * n_t * D * 4);
    L->dqm = take(H * n_t * D * 4);
    L->dkm = take(H * n_t * D * 4);
    L->dvm = take(H * n_t * D * 4);
    L->lsec = take(H * n_t * 4);
    L->dcc = take(H * n_t * 4);
    L->tlist = take(H * n_t * n_t * 4);
    L->tcount = take(H * n_t * 4);
    L->tbits = take(H * n_t * size_t((n_t + 31) / 32) * 4);
    // Split dq partials, only when the forward splits its key lists.
    const size_t items = H * n_t * size_t(info.tile_rows / 64);
    L->part_dq = take(chunks > 1 ? items * 8 * 64 * D * 4 : 0);
    L->part_dkv = take(dkdv_split(info, heads, head_dim, chunks) ? H * n_t * 8 * size_t(info.tile_rows / 32) * 2 * 32 * D * 4 : 0);
    // fp32 O_fine saved by a training forward, only when the key lists split.
    L->ofine = take(chunks > 1 ? H * S_pad * D * 4 : 0);
    L->total_bytes = off;
    L->split_chunks = int32_t(chunks);
}

namespace {

// D_t = dout[t] . O_fine[t] per tile-order row of every head, from the fp32
// O_fine a training forward saved (0 on padding rows); one thread per row,
// d in ascending order.
template <int D>
__global__ __launch_bounds__(256) void dt_kernel(const uint16_t *__restrict__ dout, const float *__restrict__ ofine,
                                                 const int32_t *__restrict__ row_src, int H, int64_t S_pad,
                                                 float *__restrict__ dt)
{
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= int64_t(H) * S_pad) return;
    const int h = int(idx / S_pad);
    const int64_t row = idx % S_pad;
    const int tok = row_src[row];
    float acc = 0.f;
    if (tok >= 0) {
        const uint16_t *g = dout + (size_t(tok) * H + h) * D;
        const float *o = ofine + size_t(idx) * D;
#pragma unroll 4
        for (int d = 0; d < D; d += 8) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(g + d);
            const float4 o0 = *reinterpret_cast<const float4 *>(o + d);
            const float4 o1 = *reinterpret_cast<const float4 *>(o + d + 4);
            acc += __uint_as_float(raw.x << 16) * o0.x;
            acc += __uint_as_float(raw.x & 0xffff0000u) * o0.y;
            acc += __uint_as_float(raw.y << 16) * o0.z;
            acc += __uint_as_float(raw.y & 0xffff0000u) * o0.w;
            acc += __uint_as_float(raw.z << 16) * o1.x;
            acc += __uint_as_float(raw.z & 0xffff0000u) * o1.y;
            acc += __uint_as_float(raw.w << 16) * o1.z;
            acc += __uint_as_float(raw.w & 0xffff0000u) * o1.w;
        }
    }
    dt[idx] = acc;
}

template <int D, int B>
void launch_bwd(const BwdArgs &a, const uint16_t *k, const uint16_t *v,
                const uint16_t *q, const uint16_t *dout, const uint16_t *gate,
                const float *o_coarse, const float *qm, const float *km, const float *vm,
                const vsa_bwd_layout &L, char *bw, float *dgate, bool split, bool ring, hipStream_t st)
{
    constexpr int HPB = 256 / D;
    const int H = a.H, n_t = a.n_t;
    const dim3 gg(n_t, (H + HPB - 1) / HPB);
    {
        KernelTimer t(K_BWD_GATHER, st);
        hipLaunchKernelGGL((frag_gather_kernel<D, B, 1>), gg, dim3(256), 0, st, v, a.row_src, a.block_len,
                           H, n_t, reinterpret_cast<uint16_t *>(bw + L.vrow));
        hipLaunchKernelGGL((frag_gather_kernel<D, B, 0>), gg, dim3(256), 0, st, k, a.row_src, a.block_len,
                           H, n_t, reinterpret_cast<uint16_t *>(bw + L.kcol));
        // Q and dO in both layouts from one read each.
        hipLaunchKernelGGL((frag_gather_kernel<D, B, 2>), gg, dim3(256), 0, st, q, a.row_src, a.block_len,
                           H, n_t, reinterpret_cast<uint16_t *>(bw + L.qrow),
                           reinterpret_cast<uint16_t *>(bw + L.qcol));
        hipLaunchKernelGGL((frag_gather_kernel<D, B, 2>), gg, dim3(256), 0, st, dout, a.row_src,
                           a.block_len, H, n_t, reinterpret_cast<uint16_t *>(bw + L.dorow),
                           reinterpret_cast<uint16_t *>(bw + L.docol));
    }
    auto *doc = reinterpret_cast<float *>(bw + L.doc);
    {
        KernelTimer t(K_BWD_PREP, st);
        hipLaunchKernelGGL((bwd_prep_kernel<D, B>), dim3(n_t, H), dim3(256), 0, st, dout, gate,
                           o_coarse, a.row_src, a.block_len, H, n_t, dgate, doc);
    }
    {
        KernelTimer t(K_BWD_COARSE, st);
        const dim3 gc((n_t + 127) / 128, H);
        hipLaunchKernelGGL((coarse_bwd_rows_kernel<D>), gc, dim3(256), 0, st, qm, km, vm, o_coarse, doc,
                           n_t, a.scale, reinterpret_cast<float *>(bw + L.lsec),
                           reinterpret_cast<float *>(bw + L.dcc), reinterpret_cast<float *>(bw + L.dqm));
        hipLaunchKernelGGL((coarse_bwd_cols_kernel<D>), gc, dim3(256), 0, st, qm, km, vm, doc,
                           reinterpret_cast<const float *>(bw + L.lsec),
                           reinterpret_cast<const float *>(bw + L.dcc), n_t, a.scale,
                           reinterpret_cast<float *>(bw + L.dkm), reinterpret_cast<float *>(bw + L.dvm));
    }
    {
        KernelTimer t(K_BWD_TLIST, st);
        const int W = (n_t + 31) / 32;
        uint32_t *tb = reinterpret_cast<uint32_t *>(bw + L.tbits);
        hipLaunchKernelGGL(tbits_kernel, dim3((n_t + 3) / 4, H), dim3(256), size_t(4) * W * 4, st, a.keep,
                           a.ref, a.P, a.n_v, n_t, a.k, a.list_len, W, tb);
        hipLaunchKernelGGL(tlist_kernel, dim3((n_t + 3) / 4, H), dim3(256), 0, st, tb, n_t, W,
                           reinterpret_cast<int32_t *>(bw + L.tlist), reinterpret_cast<int32_t *>(bw + L.tcount));
    }
    const int items = H * n_t * (B / 64);
    if (split) {
        KernelTimer t(K_BWD_DQ, st);
        hipLaunchKernelGGL((dq_kernel<D, B, true>), dim3(items * 8), dim3(64), 0, st, a);
        hipLaunchKernelGGL((dq_merge_kernel<D, B>), dim3((items * 2 * (D / 32) + 3) / 4), dim3(256), 0, st, a, items);
    } else {
        KernelTimer t(K_BWD_DQ, st);
        hipLaunchKernelGGL((dq_kernel<D, B, false>), dim3(items), dim3(64), 0, st, a);
    }
    {
        KernelTimer t(K_BWD_DKDV, st);
        if (ring) {
            hipLaunchKernelGGL((dkdv_ring_kernel<D, B>), dim3(H * n_t * 8), dim3(B * 2), (RingCfg<D, B>::LDS), st, a);
            const int units = H * n_t * (B / 32);
            hipLaunchKernelGGL((dkdv_merge_kernel<D, B>), dim3((units * 2 * (D / 32) + 3) / 4), dim3(256), 0, st, a, units);
        } else {
            hipLaunchKernelGGL((dkdv_kernel<D, B>), dim3(H * n_t), dim3(B * 2), 0, st, a);
        }
    }
}

}  // namespace
}  // namespace vsa

using namespace vsa;

extern "C" int vsa_bwd_workspace_layout(const vsa_plan_info *info, int32_t heads, int32_t head_dim,
                                        int32_t split_chunks, vsa_bwd_layout *layout)
{
    clear_error();
    if (!layout) return fail(VSA_ERR_ARG, "layout is null");
    if (int st = check_info(info)) return st;
    if (heads <= 0) return fail(VSA_ERR_ARG, "heads = %d", heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "head_dim = %d; supported: 64, 128", head_dim);
    int chunks = 0;
    if (int st = resolve_split(*info, head_dim, split_chunks, &chunks)) return st;
    compute_bwd_layout(*info, heads, head_dim, chunks, layout);
    return VSA_OK;
}

extern "C" int vsa_sparse_attn_bwd(const vsa_plan_info *info, const int32_t *row_src_dev,
                                   const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                   int32_t k_ref, int32_t k_gen, float scale, int32_t split_chunks,
                                   const void *q, const void *k, const void *v, const void *gate,
                                   const void *dout, const void *workspace, size_t workspace_bytes,
                                   const int32_t *keep_idx_dev, const float *o_coarse_dev,
                                   void *bwd_workspace, size_t bwd_workspace_bytes, float *dq,
                                   float *dk, float *dv, float *dgate, int32_t saved_stats,
                                   void *stream)
{
    clear_error();
    const char *name = "vsa_sparse_attn_bwd";
    if (int st = check_info(info)) return st;
    const bool ref = k_ref >= 0;
    if (heads <= 0) return fail(VSA_ERR_ARG, "%s: heads = %d", name, heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: head_dim = %d; supported: 64, 128", name, head_dim);
    if (k_gen < 0 || k_gen > info->n_video_tiles)
        return fail(VSA_ERR_ARG, "%s: k_gen = %d outside [0, %d]", name, k_gen, info->n_video_tiles);
    if (ref && k_ref > info->n_prefix_tiles)
        return fail(VSA_ERR_ARG, "%s: k_ref = %d outside [0, %d]", name, k_ref, info->n_prefix_tiles);
    if (!ref && info->n_prefix_tiles == 0 && k_gen == 0 && info->n_video_tiles > 0)
        return fail(VSA_ERR_ARG, "%s: empty key set: no prefix tiles and k = 0", name);
    if (ref && k_ref + k_gen == 0) return fail(VSA_ERR_ARG, "%s: empty key set: k_ref = k_gen = 0", name);
    if (!row_src_dev || !block_len_dev || !q || !k || !v || !gate || !dout || !workspace ||
        !o_coarse_dev || !bwd_workspace || !dq || !dk || !dv || !dgate)
        return fail(VSA_ERR_ARG, "%s: null device pointer", name);
    if ((ref ? k_ref + k_gen : k_gen) > 0 && !keep_idx_dev) return fail(VSA_ERR_ARG, "%s: keep_idx is null", name);
    if (!std::isfinite(scale)) return fail(VSA_ERR_ARG, "%s: scale is not finite", name);
    if (int64_t(info->rows_padded) * head_dim * 2 >= (int64_t(1) << 32))
        return fail(VSA_ERR_UNSUPPORTED, "%s: %lld padded rows x head_dim %d exceed 4 GiB per head", name,
                    (long long)info->rows_padded, head_dim);
    int chunks = 0;
    if (int st = resolve_split(*info, head_dim, split_chunks, &chunks)) return st;
    vsa_ws_layout L;
    compute_layout(*info, heads, head_dim, chunks, &L);
    if (workspace_bytes < L.total_bytes)
        return fail(VSA_ERR_ARG, "%s: workspace has %zu bytes, needs %zu", name, workspace_bytes, L.total_bytes);
    vsa_bwd_layout BL;
    compute_bwd_layout(*info, heads, head_dim, chunks, &BL);
    if (bwd_workspace_bytes < BL.total_bytes)
        return fail(VSA_ERR_ARG, "%s: backward workspace has %zu bytes, needs %zu", name,
                    bwd_workspace_bytes, BL.total_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0 || reinterpret_cast<uintptr_t>(bwd_workspace) % 256 != 0)
        return fail(VSA_ERR_ARG, "%s: workspaces must be 256-byte aligned", name);
    if (int64_t(heads) * info->n_tiles * (info->tile_rows / 32) >= (int64_t(1) << 31))
        return fail(VSA_ERR_UNSUPPORTED, "%s: too many work items", name);
    if (int st = check_device()) return st;

    const char *ws = static_cast<const char *>(workspace);
    char *bw = static_cast<char *>(bwd_workspace);
    BwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.dout = static_cast<const uint16_t *>(dout);
    a.kt = reinterpret_cast<const uint16_t *>(ws + L.k_tiled);
    a.vt = reinterpret_cast<const uint16_t *>(ws + L.v_tiled);
    a.vrow = reinterpret_cast<const uint16_t *>(bw + BL.vrow);
    a.kcol = reinterpret_cast<const uint16_t *>(bw + BL.kcol);
    a.qcol = reinterpret_cast<const uint16_t *>(bw + BL.qcol);
    a.docol = reinterpret_cast<const uint16_t *>(bw + BL.docol);
    a.qrow = reinterpret_cast<const uint16_t *>(bw + BL.qrow);
    a.dorow = reinterpret_cast<const uint16_t *>(bw + BL.dorow);
    a.kn = static_cast<const uint16_t *>(k);
    a.vn = static_cast<const uint16_t *>(v);
    a.row_src = row_src_dev;
    a.block_len = block_len_dev;
    a.keep = keep_idx_dev;
    a.tlist = reinterpret_cast<const int32_t *>(bw + BL.tlist);
    a.tcount = reinterpret_cast<const int32_t *>(bw + BL.tcount);
    a.dt = reinterpret_cast<const float *>(bw + BL.dt);
    a.dt_out = reinterpret_cast<float *>(bw + BL.dt);
    a.lse = reinterpret_cast<float *>(bw + BL.lse);
    a.dqm = reinterpret_cast<const float *>(bw + BL.dqm);
    a.dkm = reinterpret_cast<const float *>(bw + BL.dkm);
    a.dvm = reinterpret_cast<const float *>(bw + BL.dvm);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.H = heads;
    a.P = info->n_prefix_tiles;
    a.n_v = info->n_video_tiles;
    a.n_t = info->n_tiles;
    a.k = k_gen;
    a.ref = ref ? 1 : 0;
    a.list_len = ref ? k_ref + k_gen : 0;
    a.scale = scale > 0.f ? scale : 1.0f / std::sqrt(float(head_dim));
    a.scale_log2e = a.scale * 1.4426950408889634f;
    const auto *qm = reinterpret_cast<const float *>(ws + L.q_mean);
    const auto *km = reinterpret_cast<const float *>(ws + L.k_mean);
    const auto *vm = reinterpret_cast<const float *>(ws + L.v_mean);
    const auto *kk = static_cast<const uint16_t *>(k), *vv = static_cast<const uint16_t *>(v);
    const auto *qq = static_cast<const uint16_t *>(q), *dd = static_cast<const uint16_t *>(dout);
    const auto *gg = static_cast<const uint16_t *>(gate);
    a.part_dq = reinterpret_cast<float *>(bw + BL.part_dq);
    a.part_dkv = reinterpret_cast<float *>(bw + BL.part_dkv);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    // Large heads: the log-sum-exp and D_t come from the forward's split kernel
    // and a statistics merge, and dQ is split the same way; small heads
    // recompute them inside the dq kernel.
    {
        const int tb = info->tile_rows;
        const int lds = head_dim == 128 ? (tb == 64 ? ring_lds_attr<128, 64>() : ring_lds_attr<128, 128>())
                                        : (tb == 64 ? ring_lds_attr<64, 64>() : ring_lds_attr<64, 128>());
        if (lds != VSA_OK) return fail(VSA_ERR_DEVICE, "%s: cannot raise the LDS limit of the dK/dV kernel", name);
    }
    bool split = false;
    if (chunks > 1 && saved_stats) {
        // lse came with the training forward; D_t from its saved O_fine.
        const int64_t rows = int64_t(heads) * info->rows_padded;
        KernelTimer t(K_BWD_STATS, st);
        auto *dtp = reinterpret_cast<float *>(bw + BL.dt);
        auto *ofp = reinterpret_cast<const float *>(bw + BL.ofine);
        if (head_dim == 128)
            hipLaunchKernelGGL(dt_kernel<128>, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st,
                               static_cast<const uint16_t *>(dout), ofp, row_src_dev, heads,
                               int64_t(info->rows_padded), dtp);
        else
            hipLaunchKernelGGL(dt_kernel<64>, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st,
                               static_cast<const uint16_t *>(dout), ofp, row_src_dev, heads,
                               int64_t(info->rows_padded), dtp);
        split = true;
    } else if (chunks > 1) {
        const int stv = fine_stats(*info, row_src_dev, block_len_dev, heads, head_dim, chunks, ref, k_gen,
                                   ref ? k_ref : 0, a.scale, q, workspace, keep_idx_dev, dout,
                                   reinterpret_cast<float *>(bw + BL.lse),
                                   reinterpret_cast<float *>(bw + BL.dt), st);
        split = stv == VSA_OK;
    }
    const int B = info->tile_rows;
    const bool ring = dkdv_split(*info, heads, head_dim, chunks);
    if (head_dim == 128) {
        if (B == 64) launch_bwd<128, 64>(a, kk, vv, qq, dd, gg, o_coarse_dev, qm, km, vm, BL, bw, dgate, split, ring, st);
        else launch_bwd<128, 128>(a, kk, vv, qq, dd, gg, o_coarse_dev, qm, km, vm, BL, bw, dgate, split, ring, st);
    } else {
        if (B == 64) launch_bwd<64, 64>(a, kk, vv, qq, dd, gg, o_coarse_dev, qm, km, vm, BL, bw, dgate, split, ring, st);
        else launch_bwd<64, 128>(a, kk, vv, qq, dd, gg, o_coarse_dev, qm, km, vm, BL, bw, dgate, split, ring, st);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    return VSA_OK;
}

extern "C" int vsa_sparse_attn_fwd_train(const vsa_plan_info *info, const int32_t *row_src_dev,
                                         const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                         int32_t k_ref, int32_t k_gen, float scale, int32_t split_chunks,
                                         const void *q, const void *workspace, size_t workspace_bytes,
                                         const int32_t *keep_idx_dev, const float *o_coarse_dev,
                                         const void *gate, void *out, void *bwd_workspace,
                                         size_t bwd_workspace_bytes, void *stream)
{
    clear_error();
    const char *name = "vsa_sparse_attn_fwd_train";
    if (int st = check_info(info)) return st;
    if (heads <= 0) return fail(VSA_ERR_ARG, "%s: heads = %d", name, heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: head_dim = %d; supported: 64, 128", name, head_dim);
    if (!bwd_workspace) return fail(VSA_ERR_ARG, "%s: null device pointer", name);
    int chunks = 0;
    if (int st = resolve_split(*info, head_dim, split_chunks, &chunks)) return st;
    vsa_bwd_layout BL;
    compute_bwd_layout(*info, heads, head_dim, chunks, &BL);
    if (bwd_workspace_bytes < BL.total_bytes)
        return fail(VSA_ERR_ARG, "%s: backward workspace has %zu bytes, needs %zu", name,
                    bwd_workspace_bytes, BL.total_bytes);
    if (reinterpret_cast<uintptr_t>(bwd_workspace) % 256 != 0)
        return fail(VSA_ERR_ARG, "%s: workspaces must be 256-byte aligned", name);
    char *bw = static_cast<char *>(bwd_workspace);
    return fine_impl(name, info, row_src_dev, block_len_dev, heads, heads, head_dim, k_ref >= 0, false,
                     k_gen, k_ref < 0 ? 0 : k_ref, scale, split_chunks, q, workspace, workspace_bytes, keep_idx_dev,
                     o_coarse_dev, gate, out, stream, reinterpret_cast<float *>(bw + BL.lse),
                     reinterpret_cast<float *>(bw + BL.ofine));
}
