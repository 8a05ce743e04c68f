// Gate projection g = bf16(x . W_gate^T) on gfx950 MFMA.
//
// SnackOnAI analysis of ComfyUI-Ref2VA-VSA, "The Code, Annotated", snippets two
// and three: to_gate_compress is a bias-free nn.Linear whose weight is
// [heads*head_dim][hidden]; its output, viewed per head, is the kernel's
// coarse-gate input.
//
// Both operands are K-contiguous (x is [rows][hidden], W is [out][hidden]). A
// workgroup computes a 256 x 256 tile of g with 4 waves (2 x 2), each wave a
// 128 x 128 sub-tile = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 accumulated in
// fp32. 32-wide k-slices of both operands are staged in LDS with 16-byte loads
// (double buffered: the next slice is fetched into registers while the current
// one is multiplied) and read back as MFMA fragments with 16-byte LDS reads.
// Each wave loads 8 fragments per 16 products, so LDS traffic stays well under
// what the matrix cores consume.
#include <hip/hip_runtime.h>

#include "common.h"
#include "device.h"

namespace vsa {
namespace {

constexpr int BM = 256, BN = 256, BK = 32, LROW = BK + 8;  // LDS row: 80 bytes

__global__ __launch_bounds__(256) void gate_gemm_kernel(const uint16_t *__restrict__ x,
                                                       const uint16_t *__restrict__ w, int64_t M,
                                                       int N, int K, uint16_t *__restrict__ g)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LROW];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LROW];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2, l32 = lane & 31, half = lane >> 5;
    // N-blocks of one row block are consecutive, so they share the x rows in cache.
    const int nblocks = (N + BN - 1) / BN;
    const int64_t m0 = int64_t(blockIdx.x / nblocks) * BM;
    const int n0 = (blockIdx.x % nblocks) * BN;

    // Each thread moves 4 chunks of 16 bytes of x and of W per k-slice.
    uint4 ra[4], rb[4];
    auto load_global = [&](int k0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int idx = tid + 256 * t;
            const int r = idx / 4, c = idx % 4;
            const int64_t gm = m0 + r;
            const int gn = n0 + r;
            ra[t] = gm < M ? *reinterpret_cast<const uint4 *>(x + gm * K + k0 + 8 * c) : make_uint4(0, 0, 0, 0);
            rb[t] = gn < N ? *reinterpret_cast<const uint4 *>(w + int64_t(gn) * K + k0 + 8 * c)
                           : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int idx = tid + 256 * t;
            const int r = idx / 4, c = idx % 4;
            *reinterpret_cast<uint4 *>(&As[buf][r * LROW + 8 * c]) = ra[t];
            *reinterpret_cast<uint4 *>(&Bs[buf][r * LROW + 8 * c]) = rb[t];
        }
    };

    f32x16_t acc[4][4];  // [m block][n block]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    const int nk = K / BK;
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) load_global((ks + 1) * BK);
#pragma unroll
        for (int kc = 0; kc < BK / 16; ++kc) {
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = *reinterpret_cast<const bf16x8_t *>(
                    &As[buf][(wm * 128 + 32 * i + l32) * LROW + 16 * kc + 8 * half]);
                bfr[i] = *reinterpret_cast<const bf16x8_t *>(
                    &Bs[buf][(wn * 128 + 32 * i + l32) * LROW + 16 * kc + 8 * half]);
            }
            // C^T blocks: rows = n (W rows), cols = m (x rows) -> a lane owns one m.
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < nk) {
            store_lds(buf ^ 1);
            __syncthreads();
        }
    }
    // acc[i][j] element 4r + e <-> n = n0 + wn*128 + 32j + 8r + 4*half + e, m = m0 + wm*128 + 32i + l32.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + 32 * i + l32;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = n0 + wn * 128 + 32 * j + 8 * r + 4 * half;
                if (n >= N) continue;  // N is a multiple of 64, so n..n+3 are in range together
                uint2 v;
                v.x = uint32_t(f32_to_bf16(acc[i][j][4 * r + 0])) | (uint32_t(f32_to_bf16(acc[i][j][4 * r + 1])) << 16);
                v.y = uint32_t(f32_to_bf16(acc[i][j][4 * r + 2])) | (uint32_t(f32_to_bf16(acc[i][j][4 * r + 3])) << 16);
                *reinterpret_cast<uint2 *>(g + m * N + n) = v;
            }
    }
}

}  // namespace
}  // namespace vsa

using namespace vsa;

extern "C" int vsa_gate_proj(const void *x, const void *w_gate, int64_t rows, int32_t hidden,
                             int32_t out_features, void *g, void *stream)
{
    clear_error();
    if (!x || !w_gate || !g) return fail(VSA_ERR_ARG, "null device pointer");
    if (rows < 0 || hidden <= 0 || out_features <= 0)
        return fail(VSA_ERR_ARG, "bad sizes rows=%lld hidden=%d out=%d", (long long)rows, hidden,
                    out_features);
    if (hidden % 64 != 0 || out_features % 64 != 0)
        return fail(VSA_ERR_UNSUPPORTED, "hidden (%d) and out_features (%d) must be multiples of 64",
                    hidden, out_features);
    const int64_t blocks = (rows + BM - 1) / BM * ((out_features + BN - 1) / BN);
    if (blocks > 0x7fffffff) return fail(VSA_ERR_ARG, "too many rows");
    if (int st = check_device()) return st;
    if (rows == 0) return VSA_OK;
    (void)hipGetLastError();
    {
        KernelTimer t(K_GATE_GEMM, static_cast<hipStream_t>(stream));
        hipLaunchKernelGGL(gate_gemm_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(w_gate), rows, int(out_features), int(hidden),
                           static_cast<uint16_t *>(g));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return VSA_OK;
}
