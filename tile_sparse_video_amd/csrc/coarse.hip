// Coarse stage of gated, tile-sparse video attention on gfx950:
//   gather_pool  -- tile means of Q, K, V (canonical fp32 order) and K/V in tile
//                   order, fragment layout, for the fine pass (HBM-bound);
//   tile_scores  -- coarse score of every (query tile, key tile) pair of a tile
//                   range (video x video, or all x all with reference
//                   sparsity) as an fp32 fused-multiply-add chain (VALU);
//   coarse_attn  -- tile-level softmax attention over the pooled Q, K, V (fp32
//                   accumulation; products as split bf16 on the matrix cores);
//   topk         -- per score row and column group, top-k: a bitwise search for
//                   the k-th largest key over register-resident keys (a wave
//                   per row up to 2,048 columns, narrowed by a sample or a
//                   score histogram; a workgroup up to 16,384), an 8-bit radix
//                   select beyond; lowest index first on ties,
//                   ascending output.
//
// Method: SnackOnAI analysis of ComfyUI-Ref2VA-VSA ("The Code, Annotated",
// snippet two: block_len masks padding; "References": coarse tile selection
// from pooled Q/K as in the VSA paper), the Ref2VA VSA news item ("The
// two-tier attention patch": only video key tiles are pruned), and the Veda
// news item ("ComfyUI node" inputs: reference_sparsity applies the same top-k
// setting to the reference tokens).
#include <hip/hip_runtime.h>

#include <type_traits>

#include <cmath>
#include <cstring>
#include <mutex>

#include "common.h"
#include "device.h"

namespace vsa {

// ------------------------------------------------------------ device check --

int check_device()
{
    static std::mutex mu;
    static int arch_ok[64];  // 0 unknown, 1 gfx950, -1 another architecture
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VSA_ERR_DEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(VSA_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(VSA_ERR_DEVICE, "hipGetDeviceProperties failed");
        arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if (arch_ok[dev] < 0)
            return fail(VSA_ERR_UNSUPPORTED, "device %d is %s; libvsa is built for gfx950", dev,
                        prop.gcnArchName);
    }
    if (arch_ok[dev] < 0) return fail(VSA_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
    return VSA_OK;
}

namespace {

// ------------------------------------------------------------- gather/pool --
//
// One block per (tile, group of 256/D heads, tensor). The tile's real rows for
// those heads are staged in LDS (padding rows zero), each thread then owns one
// (head, d) column and sums it over the real rows in ascending row order from
// +0 (fp32 adds), dividing once by block_len. For K and V the block also
// writes the staged tile to the workspace in the MFMA fragment layout the fine
// pass streams (see vsa.h).
template <int D, int B>
__global__ __launch_bounds__(256) void gather_pool_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ row_src, const int32_t *__restrict__ block_len, int H, int ld, int n_t,
    float *__restrict__ qmean, float *__restrict__ kmean, float *__restrict__ vmean,
    uint16_t *__restrict__ kt, uint16_t *__restrict__ vt)
{
    constexpr int HPB = 256 / D;          // heads per block
    constexpr int ROW = HPB * D + 8;      // LDS row stride in bf16 (pad: 16 bytes)
    constexpr int CH = HPB * D / 8;       // 16-byte chunks per staged row
    constexpr int FR = D / 8;             // fragments per 64-row block and head
    constexpr int SUB = B / 64;
    __shared__ __attribute__((aligned(16))) uint16_t lds[B * ROW];
    __shared__ int32_t toks[B];

    const int tile = blockIdx.x;
    const int h0 = blockIdx.y * HPB;
    const int which = blockIdx.z;  // 0 = Q, 1 = K, 2 = V
    const uint16_t *X = which == 0 ? q : (which == 1 ? k : v);
    const int nh = min(HPB, H - h0);
    const int n = block_len[tile];
    const int tid = threadIdx.x;

    if (tid < B) toks[tid] = row_src[size_t(tile) * B + tid];
    __syncthreads();

    // Every load is issued unconditionally (from a clamped row, head and token,
    // so always inside the input) and masked afterwards, so a thread's loads are
    // all in flight together; a guarded load would become a branch with its own
    // wait.
    constexpr int NLD = B * CH / 256;
    uint4 val[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
        const int idx = tid + 256 * u, r = idx / CH, c = idx % CH;
        const int rr = max(min(r, n - 1), 0), hh = min(c / (D / 8), nh - 1);
        const int tok = max(toks[rr], 0);
        val[u] = *reinterpret_cast<const uint4 *>(X + (size_t(tok) * ld + h0 + hh) * D + (c % (D / 8)) * 8);
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
        const int idx = tid + 256 * u, r = idx / CH, c = idx % CH;
        const bool live = r < n && c / (D / 8) < nh;
        *reinterpret_cast<uint4 *>(&lds[r * ROW + c * 8]) = live ? val[u] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

    {
        const int hl = tid / D, d = tid % D;
        if (hl < nh) {
            float acc = 0.0f;
            for (int r = 0; r < n; ++r) acc = acc + bf16_to_f32(lds[r * ROW + tid]);
            float *mean = which == 0 ? qmean : (which == 1 ? kmean : vmean);
            mean[(size_t(h0 + hl) * n_t + tile) * D + d] = acc / float(n);
        }
    }
    if (which == 0) return;

    uint16_t *dst = which == 1 ? kt : vt;
    const int total = nh * SUB * FR * kWave;
    for (int idx = tid; idx < total; idx += 256) {
        const int lane = idx % kWave;
        const int f = (idx / kWave) % FR;
        const int sub = (idx / (kWave * FR)) % SUB;
        const int hl = idx / (kWave * FR * SUB);
        const int half = lane / 32, l32 = lane % 32;
        uint16_t e8[8];
        if (which == 1) {
            // K fragment f = kb*(D/16) + c: row 32kb + l32, d = 16c + 8*half + e.
            const int kb = f / (D / 16), c = f % (D / 16);
            const int row = 64 * sub + 32 * kb + l32;
            const uint16_t *src = &lds[row * ROW + hl * D + 16 * c + 8 * half];
            *reinterpret_cast<uint4 *>(e8) = *reinterpret_cast<const uint4 *>(src);
        } else {
            // V fragment f = db*4 + c: d = 32db + l32, row 16c + {4h..4h+3, 8+4h..8+4h+3}.
            const int db = f / 4, c = f % 4;
            const int col = hl * D + 32 * db + l32;
            const int r0 = 64 * sub + 16 * c + 4 * half;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                e8[e] = lds[(r0 + e) * ROW + col];
                e8[4 + e] = lds[(r0 + 8 + e) * ROW + col];
            }
        }
        const size_t frag = ((size_t(h0 + hl) * n_t + tile) * SUB + sub) * FR + f;
        *reinterpret_cast<uint4 *>(dst + frag * 512 + lane * 8) = *reinterpret_cast<uint4 *>(e8);
    }
}

// ------------------------------------------------------------- tile scores --
//
// scores[h][i][j] = fma-chain over ascending d of qmean[first+i][d] *
// kmean[first+j][d], from +0, for i, j < n. A block computes a 16 TM x 16 TM
// tile of (i, j) pairs; each thread owns TM x TM pairs (rows TM ty + a,
// columns tx + 16 b) and walks d in order, so every pair is the same
// sequential chain of correctly rounded fused multiply-adds. TM = 8 (128 x 128
// tiles, 4x fewer LDS reads per FMA) for large grids, TM = 4 when that would
// leave CUs idle. The means are staged in LDS 32 values of d at a time; the
// next chunk is loaded into registers (clamped rows, unconditional loads)
// while the current one is used.
template <int D, int TM>
__global__ __launch_bounds__(256, 2) void tile_scores_kernel(const float *__restrict__ qmean,
                                                         const float *__restrict__ kmean, int n_t,
                                                         int first, int n, float *__restrict__ scores)
{
    constexpr int T = 16 * TM, DC = 32, ROW = DC + 4, NCH = D / DC;
    constexpr int NL = T * DC / 4 / 256;  // float4 loads per thread per operand per chunk
    constexpr int DUN = TM == 8 ? 1 : 2;  // d-step unrolling that keeps the LDS reads in registers
    __shared__ __attribute__((aligned(16))) float qs[T * ROW];
    __shared__ __attribute__((aligned(16))) float ks[T * ROW];
    const int h = blockIdx.z;
    const int i0 = blockIdx.y * T, j0 = blockIdx.x * T;
    const int tid = threadIdx.x;
    const float *qh = qmean + (size_t(h) * n_t + first) * D;
    const float *kh = kmean + (size_t(h) * n_t + first) * D;
    // load u of a chunk: row (tid + 256 u) / 8, float4 (tid + 256 u) % 8 of the chunk
    const float *qrow[NL], *krow[NL];
    int lds_off[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int idx = tid + 256 * u, r = idx / (DC / 4), c4 = idx % (DC / 4);
        qrow[u] = qh + size_t(min(i0 + r, n - 1)) * D + 4 * c4;
        krow[u] = kh + size_t(min(j0 + r, n - 1)) * D + 4 * c4;
        lds_off[u] = r * ROW + 4 * c4;
    }
    f32x4_t qreg[NL], kreg[NL];
#define VSA_SCORES_FETCH(c)                                                                 \
    _Pragma("unroll") for (int u = 0; u < NL; ++u) {                                       \
        qreg[u] = *reinterpret_cast<const f32x4_t *>(qrow[u] + DC * (c));                  \
        kreg[u] = *reinterpret_cast<const f32x4_t *>(krow[u] + DC * (c));                  \
    }
    const int ty = tid / 16, tx = tid % 16;
    float acc[TM][TM];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = 0.0f;
    VSA_SCORES_FETCH(0)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();  // every thread is done with the previous chunk
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            *reinterpret_cast<f32x4_t *>(&qs[lds_off[u]]) = qreg[u];
            *reinterpret_cast<f32x4_t *>(&ks[lds_off[u]]) = kreg[u];
        }
        __syncthreads();
        if (c + 1 < NCH) {
            VSA_SCORES_FETCH(c + 1)
        }
#pragma unroll DUN
        for (int d = 0; d < DC; d += 4) {
            float4 qv[TM], kv[TM];
#pragma unroll
            for (int a = 0; a < TM; ++a) qv[a] = *reinterpret_cast<const float4 *>(&qs[(TM * ty + a) * ROW + d]);
#pragma unroll
            for (int b = 0; b < TM; ++b) kv[b] = *reinterpret_cast<const float4 *>(&ks[(tx + 16 * b) * ROW + d]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b) {
                    acc[a][b] = __builtin_fmaf(qv[a].x, kv[b].x, acc[a][b]);
                    acc[a][b] = __builtin_fmaf(qv[a].y, kv[b].y, acc[a][b]);
                    acc[a][b] = __builtin_fmaf(qv[a].z, kv[b].z, acc[a][b]);
                    acc[a][b] = __builtin_fmaf(qv[a].w, kv[b].w, acc[a][b]);
                }
        }
    }
    float *out = scores + size_t(h) * n * n;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int i = i0 + TM * ty + a;
        if (i >= n) continue;
#pragma unroll
        for (int b = 0; b < TM; ++b) {
            const int j = j0 + tx + 16 * b;
            if (j < n) out[size_t(i) * n + j] = acc[a][b];
        }
    }
#undef VSA_SCORES_FETCH
}

// ------------------------------------------------------- coarse attention --
//
// O_coarse[h][i] = sum_j softmax_j(scale * qmean_i . kmean_j) vmean_j over all
// n_t key tiles, for every tile i, accumulated in fp32. A workgroup of 4 waves
// covers 128 query tiles of a head; blocks of 32 key tiles (means of K and V)
// are staged in LDS once and used by all 4 waves. Each wave: S^T = K.Q^T for
// its 32 query tiles (lane = one query column), an online softmax per lane in
// fp32, then O^T += V^T.P^T.
//
// The products run on the bf16 matrix cores with split operands: every fp32
// operand x is carried as hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact
// in fp32), and a product a.b as ahi.bhi + ahi.blo + alo.bhi, accumulated in
// fp32 (the dropped alo.blo is below 2^-16 of |a b|). Three bf16 products cost
// 3/16 of an fp32 product's matrix-core cycles (v_mfma_f32_32x32x2_f32 took
// twice the time: 0.85 vs 0.43 ms at the H3-shaped layer, 7.98 vs 3.93 ms at
// the long-video one). The key blocks are staged already split and in the
// operand layouts:
//   S^T = K.Q^T (A = K: lane (key, half) holds d = 16c + 8 half + 0..7);
//   O^T += V^T.P^T (A = V^T: lane (d, half) holds the keys 16 kc + 8 (s / 4)
//   + 4 half + s % 4 of slot s, which are the S accumulator elements 8 kc + s
//   the lane holds for its query: P needs no exchange).
template <int D>
__global__ __launch_bounds__(256) void coarse_attn_kernel(const float *__restrict__ qmean,
                                                         const float *__restrict__ kmean,
                                                         const float *__restrict__ vmean, int n_t,
                                                         float scale_log2e, float *__restrict__ o_coarse)
{
    constexpr int KB = 32, NCK = D / 16, DB = D / 32;
    constexpr int KF = KB * NCK * 2 / 256;   // K fragments staged per thread
    constexpr int VF = DB * 2 * kWave / 256; // V fragments staged per thread
    static_assert(KF >= 1 && VF >= 1, "D = 64 or 128");
    __shared__ bf16x8_t khl[NCK][2][kWave];   // [chunk][hi, lo][lane]
    __shared__ bf16x8_t vhl[DB][2][2][kWave]; // [d block][key chunk][hi, lo][lane]
    const int h = blockIdx.y, wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int l32 = lane & 31, half = lane >> 5;
    const size_t hb = size_t(h) * n_t * D;
    const int qi = blockIdx.x * 128 + wave * 32 + l32;
    const bool qlive = qi < n_t;

    auto split8 = [](const float (&x)[8], bf16x8_t &hi, bf16x8_t &lo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = (__bf16)x[e];
            lo[e] = (__bf16)(x[e] - float(hi[e]));
        }
    };
    // Q (B operand of S): lane (query, half), chunk c: d = 16c + 8 half + e.
    bf16x8_t qhi[NCK], qlo[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
        float x[8];
        const float *qrow = qmean + hb + size_t(qlive ? qi : 0) * D + 16 * c + 8 * half;
        const float4 a0 = *reinterpret_cast<const float4 *>(qrow), a1 = *reinterpret_cast<const float4 *>(qrow + 4);
        x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w; x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
        if (!qlive)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        split8(x, qhi[c], qlo[c]);
    }

    f32x16_t O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = f32x16_t{};
    float mrun = -INFINITY, lrun = 0.f;

    // Staging slots. K fragment f (< 2 NCK kWave... one per (chunk, lane)):
    // key = lane % 32 of the block, d = 16 chunk + 8 (lane / 32) + 0..7.
    // V fragment f: d = 32 db + f % 32, half = (f / 32) % 2, key chunk kc =
    // (f / 64) % 2, db = f / 128; keys 16 kc + 8 (s / 4) + 4 half + s % 4.
    // The next block's values are fetched into registers under the current
    // block's products (clamped rows; rows past the end are staged as zero).
    float kx[KF][8], vx[VF][8];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < KF; ++u) {
            const int f = threadIdx.x + 256 * u, c = f / kWave, ln = f % kWave;
            const int key = ln % 32, d0 = 16 * c + 8 * (ln / 32);
            const float *row = kmean + hb + size_t(min(j0 + key, n_t - 1)) * D + d0;
            const float4 a0 = *reinterpret_cast<const float4 *>(row), a1 = *reinterpret_cast<const float4 *>(row + 4);
            kx[u][0] = a0.x; kx[u][1] = a0.y; kx[u][2] = a0.z; kx[u][3] = a0.w;
            kx[u][4] = a1.x; kx[u][5] = a1.y; kx[u][6] = a1.z; kx[u][7] = a1.w;
        }
#pragma unroll
        for (int u = 0; u < VF; ++u) {
            const int f = threadIdx.x + 256 * u;
            const int d = 32 * (f / 128) + f % 32, hf = (f / 32) % 2, kc = (f / 64) % 2;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const int key = 16 * kc + 8 * (sl / 4) + 4 * hf + sl % 4;
                vx[u][sl] = vmean[hb + size_t(min(j0 + key, n_t - 1)) * D + d];
            }
        }
    };
    fetch(0);
    for (int j0 = 0; j0 < n_t; j0 += KB) {
        __syncthreads();  // every wave is done with the previous block
#pragma unroll
        for (int u = 0; u < KF; ++u) {
            const int f = threadIdx.x + 256 * u, c = f / kWave, ln = f % kWave;
            if (j0 + ln % 32 >= n_t)
#pragma unroll
                for (int e = 0; e < 8; ++e) kx[u][e] = 0.f;
            split8(kx[u], khl[c][0][ln], khl[c][1][ln]);
        }
#pragma unroll
        for (int u = 0; u < VF; ++u) {
            const int f = threadIdx.x + 256 * u;
            const int db = f / 128, hf = (f / 32) % 2, kc = (f / 64) % 2, ln = f % 32 + 32 * hf;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl)
                if (j0 + 16 * kc + 8 * (sl / 4) + 4 * hf + sl % 4 >= n_t) vx[u][sl] = 0.f;
            split8(vx[u], vhl[db][kc][0][ln], vhl[db][kc][1][ln]);
        }
        __syncthreads();
        if (j0 + KB < n_t) fetch(j0 + KB);

        f32x16_t S = f32x16_t{};
#pragma unroll
        for (int c = 0; c < NCK; ++c) {
            const bf16x8_t kh = khl[c][0][lane], kl = khl[c][1][lane];
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qhi[c], S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qlo[c], S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qhi[c], S, 0, 0, 0);
        }
        if (j0 + KB > n_t) {  // key tiles past the end never score
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j0 + 8 * i + 4 * half + j >= n_t) S[4 * i + j] = -INFINITY;
        }
        float mx = S[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(mrun, mx);  // finite: every block has a real key tile
        const float alpha = exp2f((mrun - m_new) * scale_log2e);
        float p[16], rs = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            p[e] = exp2f((S[e] - m_new) * scale_log2e);
            rs += p[e];
        }
        rs += __shfl_xor(rs, 32);
        lrun = lrun * alpha + rs;
        mrun = m_new;
        bf16x8_t phi[2], plo[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            float x[8];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) x[sl] = p[8 * kc + sl];
            split8(x, phi[kc], plo[kc]);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[db][e] *= alpha;
        // The small terms first (vlo.phi, vhi.plo), then vhi.phi; the d blocks
        // interleaved, so consecutive products are independent.
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhl[db][kc][1][lane], phi[kc], O[db], 0, 0, 0);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhl[db][kc][0][lane], plo[kc], O[db], 0, 0, 0);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhl[db][kc][0][lane], phi[kc], O[db], 0, 0, 0);
        }
    }
    if (!qlive) return;
    // O^T[db] element 4i + j <-> d = 32db + 8i + 4*half + j, query column l32.
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            *reinterpret_cast<float4 *>(o_coarse + hb + size_t(qi) * D + d0) =
                make_float4(O[db][4 * i] * inv, O[db][4 * i + 1] * inv, O[db][4 * i + 2] * inv,
                            O[db][4 * i + 3] * inv);
        }
}

// ------------------------------------------------------------------- top-k --
//
// Per score row: the k largest of n_cols scores (columns col_first ..
// col_first + n_cols of the row), equal scores keeping the lower column,
// written as ascending ids id_first + j to out[0..k).
//
// The row's order-preserving keys stay in registers (PL per lane, read once;
// rows of up to 2,048 columns take one wave, longer ones a workgroup of up to
// eight waves, each holding a contiguous slice of the row). The k-th largest
// key T is found by a bitwise search: T is built from the top bit down,
// keeping a bit whenever at least k keys are >= the candidate. A count is one
// compare per register into a lane mask, the masks' population counts summed
// on the scalar unit (wave-uniform, no atomics, exact), plus, for a
// multi-wave row, a sum of the waves' counts through LDS. The bits above the
// highest bit in which the row's largest and smallest keys differ are common
// to every key, so the search starts below them; and as soon as exactly k
// keys are >= a candidate, those k keys are the answer and the search stops.
// Then a pass in ascending column order keeps every key > T and the first
// (k - #keys > T) keys equal to T (after an early stop: every key >= T).

// A lane mask of the wave's predicate (the compare's own result, no select).
__device__ __forceinline__ uint64_t wave_mask(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// add + the number of set bits of mask in the lanes below this one (v_mbcnt).
__device__ __forceinline__ int below_count(uint64_t mask, int add)
{
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), uint32_t(add))));
}

// Loads the keys of columns c0 + 64 e + lane. Every load is issued
// unconditionally (a clamped column for slots past the row), so all of them
// are in flight at once; a guarded load would become a branch with its own
// wait. Slots past the row hold key 0, which no count sees: every threshold
// searched is >= 1, and finite scores have keys >= 1.
template <int PL>
__device__ __forceinline__ void topk_load(const float *s, int c0, int n_cols, int lane,
                                          uint32_t (&key)[PL])
{
#pragma unroll
    for (int e = 0; e < PL; ++e) {
        const int j = c0 + kWave * e + lane;
        const uint32_t kv = score_key(s[min(j, n_cols - 1)]);
        key[e] = j < n_cols ? kv : 0u;
    }
}

// Number of this wave's keys >= t (wave-uniform).
template <int PL>
__device__ __forceinline__ int topk_count_ge(const uint32_t (&key)[PL], uint32_t t)
{
    int c = 0;
#pragma unroll
    for (int e = 0; e < PL; ++e) c += __popcll(wave_mask(key[e] >= t));
    return c;
}

// This wave's largest and smallest real key (wave-uniform).
template <int PL>
__device__ __forceinline__ void topk_range(const uint32_t (&key)[PL], int c0, int n_cols, int lane,
                                           uint32_t &kmax, uint32_t &kmin)
{
    kmax = 0u;
    kmin = 0xffffffffu;
#pragma unroll
    for (int e = 0; e < PL; ++e) {
        const bool valid = c0 + kWave * e + lane < n_cols;
        kmax = max(kmax, key[e]);
        kmin = min(kmin, valid ? key[e] : 0xffffffffu);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        kmax = max(kmax, uint32_t(__shfl_xor(int(kmax), off)));
        kmin = min(kmin, uint32_t(__shfl_xor(int(kmin), off)));
    }
    // Every lane holds the same values now. In scalar registers they keep the
    // one-wave search's candidate and loop scalar (no per-lane exec masks
    // around the loop: 6 % faster at 1,512 columns).
    kmax = uint32_t(__builtin_amdgcn_readfirstlane(int(kmax)));
    kmin = uint32_t(__builtin_amdgcn_readfirstlane(int(kmin)));
}

// The common prefix of kmax and kmin and the bit the search starts at.
__device__ __forceinline__ void topk_start(uint32_t kmax, uint32_t kmin, uint32_t &T, int &top)
{
    const uint32_t diff = kmax ^ kmin;
    top = diff == 0u ? -1 : 31 - __builtin_clz(diff);   // highest differing bit
    T = top < 0 ? kmax : kmax & ~((2u << top) - 1u);     // common prefix (2u << 31 wraps to 0)
}

// Writes this wave's selected columns in ascending order from position base.
// exact: every key >= T is selected. Otherwise every key > T, and of the keys
// equal to T the first krem of the row, eq_seen of which lie before this wave.
template <int PL>
__device__ __forceinline__ void topk_select(const uint32_t (&key)[PL], int c0, int n_cols, int lane,
                                            uint32_t T, bool exact, int krem, int base, int eq_seen,
                                            int k, int id_first, int32_t *out)
{
    if (exact) {
#pragma unroll
        for (int e = 0; e < PL; ++e) {
            if (c0 + kWave * e >= n_cols) break;  // uniform
            const int j = c0 + kWave * e + lane;
            const bool sel = j < n_cols && key[e] >= T;
            const uint64_t sel_mask = wave_mask(sel);
            const int pos = below_count(sel_mask, base);
            if (sel && pos < k) out[pos] = id_first + j;  // exactly k are selected; the bound is a guard
            base += __popcll(sel_mask);
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < PL; ++e) {
        if (c0 + kWave * e >= n_cols) break;  // uniform
        const int j = c0 + kWave * e + lane;
        const bool valid = j < n_cols;
        const bool gt = valid && key[e] > T;
        const bool eq = valid && key[e] == T;
        const uint64_t eq_mask = wave_mask(eq);
        const int eq_before = below_count(eq_mask, 0);
        const bool sel = gt || (eq && eq_seen + eq_before < krem);
        const uint64_t sel_mask = wave_mask(sel);
        const int pos = below_count(sel_mask, base);
        if (sel && pos < k) out[pos] = id_first + j;  // exactly k are selected; the bound is a guard
        base += __popcll(sel_mask);
        eq_seen += __popcll(eq_mask);
    }
}

// A threshold t >= 1 with at least r of the wave's sample registers sk (0 =
// no sample) at or above it: the r-th largest sample, or any value at which
// exactly r samples pass (the search stops there).
template <int SR>
__device__ __forceinline__ uint32_t topk_sample_threshold(const uint32_t (&sk)[SR], int r)
{
    uint32_t t = 0u;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = t | (1u << b);
        const int c = topk_count_ge<SR>(sk, cand);
        if (c >= r) t = cand;
        if (c == r) break;
    }
    return t;
}

// One wave: the k largest of m <= 64 CR candidates (cand[0..m): key, column;
// keys all >= tlo, in column order), written as ascending ids
// id_first + column to out[0..k). Every key of the row above the k-th largest
// is a candidate, so the candidates' counts are the row's.
template <int CR>
__device__ __forceinline__ void topk_finish(const uint2 *cand, int m, int k,
                                            uint32_t tlo, int lane, int id_first, int32_t *out)
{
    uint32_t ck[CR];  // candidate 64 i + lane; 0 past m
    uint32_t cmax = 0u;
#pragma unroll
    for (int i = 0; i < CR; ++i) {
        const int g = kWave * i + lane;
        const uint32_t v = cand[min(g, m - 1)].x;
        ck[i] = g < m ? v : 0u;
        cmax = max(cmax, ck[i]);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) cmax = max(cmax, uint32_t(__shfl_xor(int(cmax), off)));
    cmax = uint32_t(__builtin_amdgcn_readfirstlane(int(cmax)));
    // tlo <= the k-th largest key <= cmax: the search starts below their common prefix.
    uint32_t T;
    int top;
    topk_start(cmax, tlo, T, top);
    bool exact = false;
    for (int b = top; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        const int c = topk_count_ge<CR>(ck, cand);
        if (c >= k) T = cand;
        if (c == k) {
            exact = true;
            break;
        }
    }
    const int n_gt = exact ? k : (T == 0xffffffffu ? 0 : topk_count_ge<CR>(ck, T + 1));
    const int krem = k - n_gt;
    int obase = 0, eq_seen = 0;
#pragma unroll
    for (int i = 0; i < CR; ++i) {
        if (kWave * i >= m) break;  // uniform
        const int g = kWave * i + lane;
        const bool valid = g < m;
        const int col = int(cand[min(g, m - 1)].y);
        const bool gt = valid && (exact ? ck[i] >= T : ck[i] > T);
        const bool eq = valid && !exact && ck[i] == T;
        const uint64_t eq_mask = wave_mask(eq);
        const int eq_before = below_count(eq_mask, 0);
        const bool sel = gt || (eq && eq_seen + eq_before < krem);
        const uint64_t sel_mask = wave_mask(sel);
        const int pos = below_count(sel_mask, obase);
        if (sel && pos < k) out[pos] = id_first + col;  // exactly k are selected; the bound is a guard
        obase += __popcll(sel_mask);
        eq_seen += __popcll(eq_mask);
    }
}

constexpr int kTopkCand1 = 512;  // candidate slots per row of the one-wave sampled path
constexpr int kIcmpUge = 35;     // the compare-predicate code of unsigned >= (v_cmp_ge_u32)

// Rows of up to 64 PL columns: one wavefront per row, four rows per workgroup.
// SAMPLED (chosen on the host when k is a small share of the row): first the
// sampled path of the multi-wave kernel below, on one wave: a threshold from
// the 64 keys of four spread registers, the keys at or above it compacted in
// column order into the wave's own LDS slots (at most 512, else the full
// search runs) and the exact search and ordered selection on those alone.
template <int PL, bool SAMPLED>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores, int n_rows,
                                                   int row_len, int col_first, int n_cols, int k,
                                                   int id_first, int32_t *__restrict__ keep,
                                                   int keep_stride, int keep_first)
{
    __shared__ uint2 cand_all[SAMPLED ? 4 * (kTopkCand1 + kWave) : 1];  // per wave: candidates, then discards
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int row = blockIdx.x * 4 + wv;
    if (row >= n_rows) return;  // wave-uniform; the block has no barrier
    const float *s = scores + size_t(row) * row_len + col_first;
    int32_t *out = keep + size_t(row) * keep_stride + keep_first;
    if (k == n_cols) {
        for (int j = lane; j < n_cols; j += kWave) out[j] = id_first + j;
        return;
    }
    if (k == 0) return;
    uint32_t key[PL];
    topk_load<PL>(s, 0, n_cols, lane, key);
    if constexpr (SAMPLED) {
        static_assert(PL % 4 == 0, "the sample takes four registers");
        const int qr = lane & 3;
        uint32_t sv = key[0];
        sv = qr == 1 ? key[PL / 4] : sv;
        sv = qr == 2 ? key[PL / 2] : sv;
        sv = qr == 3 ? key[3 * PL / 4] : sv;
        const uint32_t s1[1] = {sv};
        const int ns = __popcll(wave_mask(sv != 0u));
        const float mu = float(k) * float(ns) / float(n_cols);
        const int r = int(ceilf(mu + 2.5f * sqrtf(mu))) + 1;
        if (r < ns) {  // uniform
            const uint32_t tlo = topk_sample_threshold<1>(s1, r);
            const int m = topk_count_ge<PL>(key, tlo);
            if (m >= k && m <= kTopkCand1) {  // uniform
                uint2 *cand = cand_all + wv * (kTopkCand1 + kWave);
                int base = 0;
#pragma unroll
                for (int e = 0; e < PL; ++e) {
                    const uint64_t msk = __builtin_amdgcn_uicmp(key[e], tlo, kIcmpUge);
                    const bool sel = key[e] >= tlo;
                    const int pos = below_count(msk, base);
                    cand[sel ? pos : kTopkCand1 + lane] = make_uint2(key[e], uint32_t(kWave * e + lane));
                    base += __popcll(msk);
                }
                // The wave reads back slots other lanes stored: release the
                // stores, keep the compiler from moving LDS accesses across
                // this point, then acquire (no instruction cost on one wave).
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (m <= 4 * kWave)
                    topk_finish<4>(cand, m, k, tlo, lane, id_first, out);
                else
                    topk_finish<8>(cand, m, k, tlo, lane, id_first, out);
                return;
            }
        }
    }
    uint32_t kmax, kmin, T;
    int top;
    topk_range<PL>(key, 0, n_cols, lane, kmax, kmin);
    topk_start(kmax, kmin, T, top);
    bool exact = false;  // exactly k keys are >= T
    for (int b = top; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        const int c = topk_count_ge<PL>(key, cand);
        if (c >= k) T = cand;
        if (c == k) {
            exact = true;
            break;
        }
    }
    // Without an early stop T is the k-th largest key: count(>= T) >= k >
    // count(>= T + 1); with one, the k keys >= T are the answer.
    const int n_gt = exact ? k : (T == 0xffffffffu ? 0 : topk_count_ge<PL>(key, T + 1));
    topk_select<PL>(key, 0, n_cols, lane, T, exact, k - n_gt, 0, 0, k, id_first, out);
}

// The score a key stands for (the inverse of score_key; both zeros map to +0).
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The wave's k-th largest key among its candidates ck (m of them, 0 past m; all
// inside one histogram bin, so every key of the row outside the bin is either
// above or below all of them), kk-th largest: T and whether exactly kk
// candidates are >= T. With an early stop T is raised to the candidates'
// minimum, so that "every key >= T" cannot reach below the bin.
template <int CR>
__device__ __forceinline__ void topk_bin_search(const uint32_t (&ck)[CR], int kk, uint32_t &T, bool &exact)
{
    uint32_t cmax = 0u, cmin = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < CR; ++i) {
        cmax = max(cmax, ck[i]);
        cmin = min(cmin, ck[i] == 0u ? 0xffffffffu : ck[i]);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        cmax = max(cmax, uint32_t(__shfl_xor(int(cmax), off)));
        cmin = min(cmin, uint32_t(__shfl_xor(int(cmin), off)));
    }
    cmax = uint32_t(__builtin_amdgcn_readfirstlane(int(cmax)));
    cmin = uint32_t(__builtin_amdgcn_readfirstlane(int(cmin)));
    int top;
    topk_start(cmax, cmin, T, top);
    exact = false;
    for (int b = top; b >= 0; --b) {
        const uint32_t c_t = T | (1u << b);
        const int c = topk_count_ge<CR>(ck, c_t);
        if (c >= kk) T = c_t;
        if (c == kk) {
            exact = true;
            break;
        }
    }
    if (exact) T = max(T, cmin);
}

constexpr int kHistBins = 256;

// Rows of up to 64 PL columns, one wavefront per row, when k is a large share of
// the row (the sampled path would keep too many candidates): a histogram of
// the row's scores over 256 bins of equal width between its minimum and
// maximum (LDS atomics) finds the bin that holds the k-th largest score; bin(s)
// never decreases as s grows, so every key of a higher bin is larger, and of a
// lower bin smaller, than every key of that bin. The bin's keys are compacted
// into the wave's LDS slots and the exact bitwise search runs on them alone;
// the ordered selection over the row is the full search's, so the histogram
// changes the work, never the result. Rows whose extremes are not finite, and
// bins with more than 512 keys, take the full search.
template <int PL>
__global__ __launch_bounds__(256) void topk_hist_kernel(const float *__restrict__ scores, int n_rows,
                                                        int row_len, int col_first, int n_cols, int k,
                                                        int id_first, int32_t *__restrict__ keep,
                                                        int keep_stride, int keep_first)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][kHistBins + 4];  // + a bin for padding
    __shared__ uint2 cand_all[4 * (kTopkCand1 + kWave)];  // per wave: candidates, then discards
    // The wave index through readfirstlane: the row, its base and its output
    // are then scalar, and the loads take a 32-bit offset from a scalar base.
    const int lane = threadIdx.x % kWave, wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int row = blockIdx.x * 4 + wv;
    if (row >= n_rows) return;  // wave-uniform; the block has no barrier
    const float *s = scores + size_t(row) * row_len + col_first;
    int32_t *out = keep + size_t(row) * keep_stride + keep_first;
    if (k == n_cols) {
        for (int j = lane; j < n_cols; j += kWave) out[j] = id_first + j;
        return;
    }
    if (k == 0) return;
    uint32_t key[PL];
    float sc[PL];  // the scores themselves (clamped column past the row)
#pragma unroll
    for (int e = 0; e < PL; ++e) {
        const unsigned j = min(unsigned(kWave * e + lane), unsigned(n_cols - 1));
        sc[e] = s[j];
        key[e] = kWave * e + lane < n_cols ? score_key(sc[e]) : 0u;
    }
    uint32_t kmax, kmin, T;
    int top;
    topk_range<PL>(key, 0, n_cols, lane, kmax, kmin);
    const float fmin = key_value(kmin), fmax = key_value(kmax);
    const float span = fmax - fmin;
    const float inv = float(kHistBins) / span;
    // Finiteness from the exponent bits (the build does not honour NaNs in
    // floating-point tests).
    auto finite = [](float f) { return (__float_as_uint(f) & 0x7f800000u) != 0x7f800000u; };
    if (kmax != kmin && finite(fmin) && finite(fmax) && finite(span) && finite(inv) && span > 0.f) {  // uniform
        uint32_t *hist = hist_all[wv];
        // (s - fmin) >= 0 and <= span, times inv, is finite and at most ~256:
        // truncation gives a bin that never decreases as s grows.
        // The bin of a real key's score (a zero of either sign reads as +0, as
        // its key does: the key order ignores the sign of zero).
        auto bin_of = [&](float v) -> int { return min(kHistBins - 1, int((v - fmin) * inv)); };
        int bins[PL];
#pragma unroll
        for (int e = 0; e < PL; ++e) {
            const int bn = bin_of(sc[e]);
            bins[e] = kWave * e + lane < n_cols ? bn : kHistBins;
        }
        reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int e = 0; e < PL; ++e) atomicAdd(&hist[bins[e]], 1u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Lane l holds bins 4l .. 4l + 3; suf = keys in bins >= 4l (inclusive
        // suffix over lanes). suf of lane 0 is the row's count, >= k.
        const uint4 hv = reinterpret_cast<const uint4 *>(hist)[lane];
        int suf = int(hv.x + hv.y + hv.z + hv.w);
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_down(suf, off);
            if (lane + off < kWave) suf += v;
        }
        const uint64_t ge = wave_mask(suf >= k);  // lanes 0 .. L, L the last with suf >= k
        const int L = 63 - __builtin_clzll(ge);
        const int h0 = __builtin_amdgcn_readlane(int(hv.x), L), h1 = __builtin_amdgcn_readlane(int(hv.y), L);
        const int h2 = __builtin_amdgcn_readlane(int(hv.z), L), h3 = __builtin_amdgcn_readlane(int(hv.w), L);
        int above = __builtin_amdgcn_readlane(suf, L) - (h0 + h1 + h2 + h3);  // keys in bins > 4L + 3
        int bstar, m;
        if (above + h3 >= k) {
            bstar = 4 * L + 3;
            m = h3;
        } else if (above + h3 + h2 >= k) {
            above += h3;
            bstar = 4 * L + 2;
            m = h2;
        } else if (above + h3 + h2 + h1 >= k) {
            above += h3 + h2;
            bstar = 4 * L + 1;
            m = h1;
        } else {
            above += h3 + h2 + h1;
            bstar = 4 * L;
            m = h0;
        }
        if (m <= kTopkCand1) {  // uniform
            uint2 *cand = cand_all + wv * (kTopkCand1 + kWave);
            int base = 0;
#pragma unroll
            for (int e = 0; e < PL; ++e) {
                const bool sel = bins[e] == bstar;
                const uint64_t msk = wave_mask(sel);
                const int pos = below_count(msk, base);
                cand[sel ? pos : kTopkCand1 + lane] = make_uint2(key[e], uint32_t(kWave * e + lane));
                base += __popcll(msk);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int kk = k - above;  // 1 <= kk <= m
            bool exact;
            int n_gt;
            auto finish = [&](auto cr_tag) {
                constexpr int CR = decltype(cr_tag)::value;
                uint32_t ck[CR];
#pragma unroll
                for (int i = 0; i < CR; ++i) {
                    const int g = kWave * i + lane;
                    const uint32_t v = cand[min(g, m - 1)].x;
                    ck[i] = g < m ? v : 0u;
                }
                topk_bin_search<CR>(ck, kk, T, exact);
                n_gt = exact ? k : above + topk_count_ge<CR>(ck, T + 1);
            };
            if (m <= kWave) finish(std::integral_constant<int, 1>{});
            else if (m <= 4 * kWave) finish(std::integral_constant<int, 4>{});
            else finish(std::integral_constant<int, 8>{});
            topk_select<PL>(key, 0, n_cols, lane, T, exact, k - n_gt, 0, 0, k, id_first, out);
            return;
        }
    }
    topk_start(kmax, kmin, T, top);
    bool exact = false;
    for (int b = top; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        const int c = topk_count_ge<PL>(key, cand);
        if (c >= k) T = cand;
        if (c == k) {
            exact = true;
            break;
        }
    }
    const int n_gt = exact ? k : (T == 0xffffffffu ? 0 : topk_count_ge<PL>(key, T + 1));
    topk_select<PL>(key, 0, n_cols, lane, T, exact, k - n_gt, 0, 0, k, id_first, out);
}

constexpr int kTopkMaxWaves = 8;
constexpr int kTopkCand = 1024;  // candidate slots of the sampled path (16 per lane of one wave)

// Rows of up to 64 PL W columns: one workgroup of W = blockDim.x / 64 waves per
// row, wave w holding columns [64 PL w, 64 PL (w + 1)).
//
// Sampled path (taken when it applies): a full-row bitwise search costs one
// workgroup barrier and a count of every key per bit, and the kernel's time
// follows the instructions it issues. So first a threshold t is taken from a
// sample of 64 W keys (four registers of every wave, so the sample spans the
// row): the r-th largest sample, with r above the sample's expected count of
// keys >= the k-th largest by 2.5 standard deviations plus one. Then one
// count of the keys >= t over the row; if there are m with k <= m <= 1,024
// (else the full search below runs), the k-th largest key is among them: they
// are compacted in column order into LDS and one wave finishes the exact
// search and the ordered selection on them alone. The sample only decides how
// much work is left, never the result.
//
// Full search: counts are summed across the waves through LDS, one barrier per
// search step (two buffers alternate, so a buffer is rewritten only after every
// wave has passed the barrier that follows its reads). Every branch taken on a
// count is uniform over the workgroup.
template <int PL>
__global__ __launch_bounds__(kWave * kTopkMaxWaves) void topk_wide_kernel(
    const float *__restrict__ scores, int n_rows, int row_len, int col_first, int n_cols, int k,
    int id_first, int32_t *__restrict__ keep, int keep_stride, int keep_first)
{
    static_assert(PL % 4 == 0, "the sample takes four registers per wave");
    if (int(blockIdx.x) >= n_rows) return;  // one workgroup per row (the grid has n_rows)
    __shared__ int xs[2][kTopkMaxWaves];
    __shared__ uint32_t xmax[kTopkMaxWaves], xmin[kTopkMaxWaves];
    __shared__ uint32_t samp[kTopkMaxWaves * kWave];
    __shared__ uint2 cand[kTopkCand + kWave];  // (key, column); the last 64: discarded stores
    __shared__ uint32_t s_tlo;
    const int W = blockDim.x / kWave;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int row = blockIdx.x;
    const float *s = scores + size_t(row) * row_len + col_first;
    int32_t *out = keep + size_t(row) * keep_stride + keep_first;
    if (k == n_cols) {
        for (int j = threadIdx.x; j < n_cols; j += blockDim.x) out[j] = id_first + j;
        return;
    }
    if (k == 0) return;
    const int c0 = w * PL * kWave;
    uint32_t key[PL];
    topk_load<PL>(s, c0, n_cols, lane, key);
    // Publishes this wave's value v and returns the values' sum over the
    // waves before this one (before) and over all waves.
    int par = 0;
    auto exchange = [&](int v, int &before) -> int {
        if (lane == 0) xs[par][w] = v;
        __syncthreads();
        int all = 0;
        before = 0;
        for (int i = 0; i < W; ++i) {
            const int x = xs[par][i];
            before += i < w ? x : 0;
            all += x;
        }
        par ^= 1;
        return all;
    };
    int before;

    // ---- Sampled path.
    {
        // Lane l offers register (l % 4) PL / 4: columns from all four quarters of the slice.
        const int qr = lane & 3;
        uint32_t sv = key[0];
        sv = qr == 1 ? key[PL / 4] : sv;
        sv = qr == 2 ? key[PL / 2] : sv;
        sv = qr == 3 ? key[3 * PL / 4] : sv;
        samp[w * kWave + lane] = sv;  // 0 past the row: never counted
    }
    __syncthreads();
    if (w == 0) {
        uint32_t sk[kTopkMaxWaves];
        int ns = 0;
#pragma unroll
        for (int i = 0; i < kTopkMaxWaves; ++i) {
            const uint32_t v = samp[min(i, W - 1) * kWave + lane];
            sk[i] = i < W ? v : 0u;
            ns += __popcll(wave_mask(sk[i] != 0u));
        }
        const float mu = float(k) * float(ns) / float(n_cols);
        const int r = int(ceilf(mu + 2.5f * sqrtf(mu))) + 1;
        uint32_t t = 0u;  // 0: no threshold (the full search runs)
        if (r < ns) {
            // Only the registers that hold samples are searched.
            if (W <= 2) {
                const uint32_t s2[2] = {sk[0], sk[1]};
                t = topk_sample_threshold<2>(s2, r);
            } else if (W <= 4) {
                const uint32_t s4[4] = {sk[0], sk[1], sk[2], sk[3]};
                t = topk_sample_threshold<4>(s4, r);
            } else {
                t = topk_sample_threshold<kTopkMaxWaves>(sk, r);
            }
        }
        if (lane == 0) s_tlo = t;
    }
    __syncthreads();
    const uint32_t tlo = uint32_t(__builtin_amdgcn_readfirstlane(int(s_tlo)));
    if (tlo != 0u) {
        const int m = __builtin_amdgcn_readfirstlane(exchange(topk_count_ge<PL>(key, tlo), before));
        if (m >= k && m <= kTopkCand) {  // uniform over the workgroup
            // Every key >= tlo, in column order (slots past the row hold 0 < tlo).
            // Every lane stores (no branch around the store): the unselected
            // ones into a slot of their own past the candidates.
            int base = __builtin_amdgcn_readfirstlane(before);
#pragma unroll
            for (int e = 0; e < PL; ++e) {
                const uint64_t msk = __builtin_amdgcn_uicmp(key[e], tlo, kIcmpUge);  // the compare's own lane mask
                const bool sel = key[e] >= tlo;
                const int pos = below_count(msk, base);
                cand[sel ? pos : kTopkCand + lane] = make_uint2(key[e], uint32_t(c0 + kWave * e + lane));
                base += __popcll(msk);
            }
            __syncthreads();
            if (w != 0) return;
            // Registers for the candidates actually present (a uniform choice).
            if (m <= 4 * kWave)
                topk_finish<4>(cand, m, k, tlo, lane, id_first, out);
            else if (m <= 8 * kWave)
                topk_finish<8>(cand, m, k, tlo, lane, id_first, out);
            else if (m <= 12 * kWave)
                topk_finish<12>(cand, m, k, tlo, lane, id_first, out);
            else
                topk_finish<kTopkCand / kWave>(cand, m, k, tlo, lane, id_first, out);
            return;
        }
    }

    // ---- Full search.
    uint32_t kmax, kmin, T;
    int top;
    topk_range<PL>(key, c0, n_cols, lane, kmax, kmin);
    if (lane == 0) {
        xmax[w] = kmax;
        xmin[w] = kmin;
    }
    __syncthreads();
    for (int i = 0; i < W; ++i) {
        kmax = max(kmax, xmax[i]);
        kmin = min(kmin, xmin[i]);
    }
    topk_start(kmax, kmin, T, top);
    bool exact = false;
    for (int b = top; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        const int c = exchange(topk_count_ge<PL>(key, cand), before);
        if (c >= k) T = cand;
        if (c == k) {
            exact = true;
            break;
        }
    }
    if (exact) {
        exchange(topk_count_ge<PL>(key, T), before);
        topk_select<PL>(key, c0, n_cols, lane, T, true, 0, before, 0, k, id_first, out);
        return;
    }
    // gt and eq counts packed in one word (each below 2^16: n_cols <= 16,384).
    const int gt = T == 0xffffffffu ? 0 : topk_count_ge<PL>(key, T + 1);
    const int ge = topk_count_ge<PL>(key, T);
    const int all = exchange(gt | ((ge - gt) << 16), before);
    const int krem = k - (all & 0xffff);
    const int gt_before = before & 0xffff, eq_before = before >> 16;
    topk_select<PL>(key, c0, n_cols, lane, T, false, krem, gt_before + min(eq_before, krem),
                    eq_before, k, id_first, out);
}

// Rows beyond 16,384 columns: a four-pass 8-bit radix select over LDS
// histograms, re-reading the row (from L2) in each pass in batches of
// kRadixBatch loads per lane, then the same ordered compaction.
constexpr int kRadixBatch = 8;
__global__ __launch_bounds__(256) void topk_radix_kernel(const float *__restrict__ scores,
                                                         int n_rows, int row_len, int col_first,
                                                         int n_cols, int k, int id_first,
                                                         int32_t *__restrict__ keep, int keep_stride,
                                                         int keep_first)
{
    __shared__ uint32_t hist[4][256];
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int row = blockIdx.x * 4 + w;
    const bool live = row < n_rows;
    const float *s = scores + size_t(live ? row : 0) * row_len + col_first;
    int32_t *out = keep + size_t(live ? row : 0) * keep_stride + keep_first;
    if (k == n_cols) {  // uniform across the launch
        if (live)
            for (int j = lane; j < n_cols; j += kWave) out[j] = id_first + j;
        return;
    }
    uint32_t prefix = 0, mask = 0;
    int krem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int b = 0; b < 4; ++b) hist[w][4 * lane + b] = 0;
        __syncthreads();
        if (live)
            for (int j0 = 0; j0 < n_cols; j0 += kRadixBatch * kWave) {
                uint32_t kb[kRadixBatch];
#pragma unroll
                for (int u = 0; u < kRadixBatch; ++u)
                    kb[u] = score_key(s[min(j0 + kWave * u + lane, n_cols - 1)]);
#pragma unroll
                for (int u = 0; u < kRadixBatch; ++u)
                    if (j0 + kWave * u + lane < n_cols && (kb[u] & mask) == prefix)
                        atomicAdd(&hist[w][(kb[u] >> shift) & 255u], 1u);
            }
        __syncthreads();
        // Lane L owns digits 255-4L .. 252-4L (descending); an inclusive scan over
        // lanes gives the number of matching keys at or above each lane's digits.
        uint32_t c[4], local = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            c[b] = hist[w][255 - 4 * lane - b];
            local += c[b];
        }
        uint32_t incl = local;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const uint32_t excl = incl - local;
        const bool mine = excl < uint32_t(krem) && uint32_t(krem) <= incl;
        int digit = 0;
        uint32_t above = excl;
        if (mine) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (above + c[b] >= uint32_t(krem)) {
                    digit = 255 - 4 * lane - b;
                    break;
                }
                above += c[b];
            }
        }
        const uint64_t who = wave_mask(mine);
        const int src = who ? __ffsll((unsigned long long)who) - 1 : 0;
        digit = __shfl(digit, src);
        above = __shfl(above, src);
        krem -= int(above);
        prefix |= uint32_t(digit) << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    if (!live || k == 0) return;
    // prefix is the k-th largest key; keep krem of the keys equal to it.
    int base = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n_cols; j0 += kRadixBatch * kWave) {
        uint32_t kb[kRadixBatch];
#pragma unroll
        for (int u = 0; u < kRadixBatch; ++u)
            kb[u] = score_key(s[min(j0 + kWave * u + lane, n_cols - 1)]);
#pragma unroll
        for (int u = 0; u < kRadixBatch; ++u) {
            const int j = j0 + kWave * u + lane;
            const bool valid = j < n_cols;
            const bool gt = valid && kb[u] > prefix;
            const bool eq = valid && kb[u] == prefix;
            const uint64_t eq_mask = wave_mask(eq);
            const int eq_before = below_count(eq_mask, 0);
            const bool sel = gt || (eq && eq_seen + eq_before < krem);
            const uint64_t sel_mask = wave_mask(sel);
            const int pos = below_count(sel_mask, base);
            if (sel && pos < k) out[pos] = id_first + j;  // exactly k are selected; the bound is a guard
            base += __popcll(sel_mask);
            eq_seen += __popcll(eq_mask);
        }
    }
}

// Top-k of one column group for n_rows rows.
void launch_topk(const float *scores, int n_rows, int row_len, int col_first, int n_cols, int k,
                 int id_first, int32_t *keep, int keep_stride, int keep_first, hipStream_t st)
{
    if (n_rows == 0 || n_cols == 0) return;
    KernelTimer t(K_TOPK, st);
    // The one-wave sampled path pays when the candidates it expects (the
    // sample rank it thresholds at, scaled to the row) fit its 512 slots with
    // room to spare; otherwise rows of 8 or more keys per lane take the
    // histogram path (0.155 -> 0.131 ms at the H3-shaped layer; at the
    // Veda-style layer's k / n = 10 % it was 4 % slower than the sampled path),
    // and shorter rows the plain search.
    const double mu = 64.0 * k / n_cols;
    const bool sampled = n_cols >= 8 * kWave && k < n_cols &&
                         (std::ceil(mu + 2.5 * std::sqrt(mu)) + 1.0) * n_cols / kWave <= 0.8 * kTopkCand1;
#define VSA_TOPK(PLV)                                                                                  \
    do {                                                                                               \
        if (sampled && (PLV) % 4 == 0 && (PLV) >= 8)                                                   \
            hipLaunchKernelGGL((topk_kernel<PLV, (PLV) % 4 == 0 && (PLV) >= 8>), dim3((n_rows + 3) / 4), \
                               dim3(256), 0, st, scores, n_rows, row_len, col_first, n_cols, k,        \
                               id_first, keep, keep_stride, keep_first);                               \
        else if ((PLV) % 4 == 0 && (PLV) >= 8)                                                        \
            hipLaunchKernelGGL((topk_hist_kernel<((PLV) % 4 == 0 ? (PLV) : 8)>), dim3((n_rows + 3) / 4), \
                               dim3(256), 0, st, scores, n_rows, row_len, col_first, n_cols, k,        \
                               id_first, keep, keep_stride, keep_first);                               \
        else                                                                                           \
            hipLaunchKernelGGL((topk_kernel<PLV, false>), dim3((n_rows + 3) / 4), dim3(256), 0, st,     \
                               scores, n_rows, row_len, col_first, n_cols, k, id_first, keep,          \
                               keep_stride, keep_first);                                               \
    } while (0)
#define VSA_TOPK_WIDE(PLV)                                                                         \
    hipLaunchKernelGGL(topk_wide_kernel<PLV>, dim3(n_rows),                                        \
                       dim3(kWave * ((n_cols + kWave * (PLV)-1) / (kWave * (PLV)))), 0, st, scores, \
                       n_rows, row_len, col_first, n_cols, k, id_first, keep, keep_stride,         \
                       keep_first)
    if (n_cols <= 4 * kWave) VSA_TOPK(4);
    else if (n_cols <= 8 * kWave) VSA_TOPK(8);
    else if (n_cols <= 12 * kWave) VSA_TOPK(12);
    else if (n_cols <= 16 * kWave) VSA_TOPK(16);
    else if (n_cols <= 24 * kWave) VSA_TOPK(24);
    else if (n_cols <= 32 * kWave) VSA_TOPK(32);
    else if (n_cols <= 24 * kWave * kTopkMaxWaves) VSA_TOPK_WIDE(24);
    else if (n_cols <= 32 * kWave * kTopkMaxWaves) VSA_TOPK_WIDE(32);
    else
        hipLaunchKernelGGL(topk_radix_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, st, scores,
                           n_rows, row_len, col_first, n_cols, k, id_first, keep, keep_stride,
                           keep_first);
#undef VSA_TOPK
#undef VSA_TOPK_WIDE
}

template <int D, int B>
void launch_gather_pool(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *row_src,
                        const int32_t *block_len, int H, int ld, int n_t, float *qm, float *km, float *vm,
                        uint16_t *kt, uint16_t *vt, hipStream_t st)
{
    constexpr int HPB = 256 / D;
    dim3 grid(n_t, (H + HPB - 1) / HPB, 3);
    KernelTimer t(K_GATHER_POOL, st);
    hipLaunchKernelGGL((gather_pool_kernel<D, B>), grid, dim3(256), 0, st, q, k, v, row_src,
                       block_len, H, ld, n_t, qm, km, vm, kt, vt);
}

// Scores over tiles [first, first + n) x [first, first + n), then the coarse
// attention over all tiles.
template <int D>
void launch_coarse(const vsa_plan_info &info, int H, float scale, const float *qm, const float *km,
                   const float *vm, int first, int n, float *scores, float *o_coarse, hipStream_t st)
{
    const int n_t = info.n_tiles;
    if (n > 0) {
        KernelTimer t(K_VIDEO_SCORES, st);
        const int64_t big = int64_t((n + 127) / 128) * ((n + 127) / 128) * H;
        if (big >= 512) {
            dim3 grid((n + 127) / 128, (n + 127) / 128, H);
            hipLaunchKernelGGL((tile_scores_kernel<D, 8>), grid, dim3(256), 0, st, qm, km, n_t, first, n, scores);
        } else {
            dim3 grid((n + 63) / 64, (n + 63) / 64, H);
            hipLaunchKernelGGL((tile_scores_kernel<D, 4>), grid, dim3(256), 0, st, qm, km, n_t, first, n, scores);
        }
    }
    dim3 grid2((n_t + 127) / 128, H);
    KernelTimer t(K_COARSE_ATTN, st);
    hipLaunchKernelGGL((coarse_attn_kernel<D>), grid2, dim3(256), 0, st, qm, km, vm, n_t,
                       scale * 1.4426950408889634f, o_coarse);
}

}  // namespace

// Shared body of the coarse entry points. ref: reference-sparsity mode
// (scores over all tiles, two selections per query tile); otherwise the
// default mode (video x video scores, k_gen video tiles per video query tile).
// ld: heads per token row of q, k, v (the pointers address the first head).
int coarse_impl(const char *name, const vsa_plan_info *info, const int32_t *row_src_dev,
                const int32_t *block_len_dev, int heads, int ld, int head_dim, bool ref, double sparsity,
                int64_t keep_k, double ref_sparsity, int64_t ref_keep_k, float scale, const void *q,
                const void *k, const void *v, void *workspace, size_t workspace_bytes,
                int32_t *keep_idx_dev, float *o_coarse_dev, void *stream)
{
    if (int st = check_info(info)) return st;
    if (heads <= 0 || ld < heads) return fail(VSA_ERR_ARG, "%s: heads = %d (row stride %d)", name, heads, ld);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: head_dim = %d; supported: 64, 128", name, head_dim);
    // q = k = v = null: the workspace already holds the tiled K/V and the tile
    // means (written by the chunked producer), so the gather is skipped.
    const bool pretiled = !q && !k && !v;
    if (!row_src_dev || !block_len_dev || !workspace || !o_coarse_dev || (!pretiled && (!q || !k || !v)))
        return fail(VSA_ERR_ARG, "%s: null device pointer", name);
    if (!(std::isfinite(scale))) return fail(VSA_ERR_ARG, "%s: scale is not finite", name);
    int32_t k_gen = 0, k_ref = 0;
    if (int st = vsa_keep_count(info, sparsity, keep_k, &k_gen)) return st;
    if (ref)
        if (int st = vsa_ref_keep_count(info, ref_sparsity, ref_keep_k, &k_ref)) return st;
    if (k_gen + k_ref > 0 && !keep_idx_dev)
        return fail(VSA_ERR_ARG, "%s: keep_idx is null with %d kept tiles per row", name, k_gen + k_ref);
    // The coarse stage writes only the regions ahead of the fine-pass partials,
    // which do not depend on the split count.
    vsa_ws_layout L;
    compute_layout(*info, heads, head_dim, 1, &L);
    if (workspace_bytes < L.part_o)
        return fail(VSA_ERR_ARG, "%s: workspace has %zu bytes, needs %zu", name, workspace_bytes, L.part_o);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(VSA_ERR_ARG, "%s: workspace must be 256-byte aligned", name);
    if (int st = check_device()) return st;

    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(float(head_dim));
    char *ws = static_cast<char *>(workspace);
    auto *qm = reinterpret_cast<float *>(ws + L.q_mean);
    auto *km = reinterpret_cast<float *>(ws + L.k_mean);
    auto *vm = reinterpret_cast<float *>(ws + L.v_mean);
    auto *kt = reinterpret_cast<uint16_t *>(ws + L.k_tiled);
    auto *vt = reinterpret_cast<uint16_t *>(ws + L.v_tiled);
    auto *sc_buf = reinterpret_cast<float *>(ws + L.scores);
    auto *qq = static_cast<const uint16_t *>(q);
    auto *kk_ = static_cast<const uint16_t *>(k);
    auto *vv = static_cast<const uint16_t *>(v);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int n_t = info->n_tiles, B = info->tile_rows, P = info->n_prefix_tiles;
    const int n_v = info->n_video_tiles;
    const int first = ref ? 0 : P, n = ref ? n_t : n_v;

    (void)hipGetLastError();
    if (head_dim == 128) {
        if (pretiled) {
        } else if (B == 64) launch_gather_pool<128, 64>(qq, kk_, vv, row_src_dev, block_len_dev, heads, ld, n_t, qm, km, vm, kt, vt, st);
        else launch_gather_pool<128, 128>(qq, kk_, vv, row_src_dev, block_len_dev, heads, ld, n_t, qm, km, vm, kt, vt, st);
        launch_coarse<128>(*info, heads, sc, qm, km, vm, first, n, sc_buf, o_coarse_dev, st);
    } else {
        if (pretiled) {
        } else if (B == 64) launch_gather_pool<64, 64>(qq, kk_, vv, row_src_dev, block_len_dev, heads, ld, n_t, qm, km, vm, kt, vt, st);
        else launch_gather_pool<64, 128>(qq, kk_, vv, row_src_dev, block_len_dev, heads, ld, n_t, qm, km, vm, kt, vt, st);
        launch_coarse<64>(*info, heads, sc, qm, km, vm, first, n, sc_buf, o_coarse_dev, st);
    }
    if (!ref) {
        launch_topk(sc_buf, heads * n_v, n_v, 0, n_v, k_gen, P, keep_idx_dev, k_gen, 0, st);
    } else {
        const int Lk = k_ref + k_gen;
        launch_topk(sc_buf, heads * n_t, n_t, 0, P, k_ref, 0, keep_idx_dev, Lk, 0, st);
        launch_topk(sc_buf, heads * n_t, n_t, P, n_v, k_gen, P, keep_idx_dev, Lk, k_ref, st);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    return VSA_OK;
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_coarse_topk(const vsa_plan_info *info, const int32_t *row_src_dev,
                               const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                               double sparsity, int64_t keep_k, float scale, const void *q,
                               const void *k, const void *v, void *workspace, size_t workspace_bytes,
                               int32_t *keep_idx_dev, float *o_coarse_dev, void *stream)
{
    clear_error();
    return coarse_impl("vsa_coarse_topk", info, row_src_dev, block_len_dev, heads, heads, head_dim, false,
                       sparsity, keep_k, 0.0, -1, scale, q, k, v, workspace, workspace_bytes,
                       keep_idx_dev, o_coarse_dev, stream);
}

extern "C" int vsa_coarse_topk_ref(const vsa_plan_info *info, const int32_t *row_src_dev,
                                   const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                   double sparsity, int64_t keep_k, double ref_sparsity,
                                   int64_t ref_keep_k, float scale, const void *q, const void *k,
                                   const void *v, void *workspace, size_t workspace_bytes,
                                   int32_t *keep_idx_dev, float *o_coarse_dev, void *stream)
{
    clear_error();
    return coarse_impl("vsa_coarse_topk_ref", info, row_src_dev, block_len_dev, heads, heads, head_dim, true,
                       sparsity, keep_k, ref_sparsity, ref_keep_k, scale, q, k, v, workspace,
                       workspace_bytes, keep_idx_dev, o_coarse_dev, stream);
}
