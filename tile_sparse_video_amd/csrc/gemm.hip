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
// fp32. 64-wide k-slices of both operands are staged in LDS (double buffered,
// 144 KB): the next slice is fetched into registers with bounds-checked
// buffer loads (rows past the end read as zero) while the current one is
// multiplied, and within a slice the MFMA fragments of the next 16-wide step
// are read from LDS while the current step's 16 products run.
#include <hip/hip_runtime.h>

#include "common.h"
#include "device.h"

namespace vsa {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, LROW = BK + 8;  // LDS row: 144 bytes
constexpr int KC = BK / 16;                                 // MFMA k-steps per slice
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource word 3, 32-bit data (gfx9 family)

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

__global__ __launch_bounds__(256, 1) void gate_gemm_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w, int64_t M,
                                                          int N, int K, uint16_t *__restrict__ g)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t *As = lds;                   // [2][BM][LROW]
    uint16_t *Bs = lds + 2 * BM * LROW;   // [2][BN][LROW]
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2, l32 = lane & 31, half = lane >> 5;
    // N-blocks of one row block are consecutive, so they share the x rows in cache.
    const int nblocks = (N + BN - 1) / BN;
    const int mb = __builtin_amdgcn_readfirstlane(int(blockIdx.x) / nblocks);
    const int64_t m0 = int64_t(mb) * BM;
    const int n0 = __builtin_amdgcn_readfirstlane(int(blockIdx.x) - mb * nblocks) * BN;

    // One buffer resource per operand, based at the tile's first row and sized
    // to the rows that exist, so loads past the last row return zero.
    const uint32_t row_bytes = uint32_t(K) * 2;
    const int64_t m_left = M - m0;
    const uint32_t a_rows = __builtin_amdgcn_readfirstlane(m_left < BM ? int(m_left) : BM);
    const uint32_t b_rows = __builtin_amdgcn_readfirstlane(min(N - n0, BN));
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + m0 * K), (short)0, a_rows * row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + int64_t(n0) * K), (short)0, b_rows * row_bytes, kRsrcWord3);

    // Each thread moves 8 chunks of 16 bytes of x and of W per k-slice: chunk
    // idx = tid + 256 t covers row idx / 8, bytes 16 (idx % 8) of the slice.
    u32x4_t pa[8], pb[8];
    auto load_global = [&](int k0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int idx = tid + 256 * t;
            const uint32_t off = uint32_t(idx / 8) * row_bytes + uint32_t(k0) * 2 + 16 * (idx % 8);
            pa[t] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
            pb[t] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int idx = tid + 256 * t;
            const int r = idx / 8, c = idx % 8;
            *reinterpret_cast<u32x4_t *>(&As[(buf * BM + r) * LROW + 8 * c]) = pa[t];
            *reinterpret_cast<u32x4_t *>(&Bs[(buf * BN + r) * LROW + 8 * c]) = pb[t];
        }
    };
    // Fragments of k-step kc: lane -> row 32 i + l32 of the wave's 128 rows,
    // reduction slots 16 kc + 8 half .. +7.
    auto load_frags = [&](int buf, int kc, bf16x8_t (&af)[4], bf16x8_t (&bf)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = *reinterpret_cast<const bf16x8_t *>(
                &As[(buf * BM + wm * 128 + 32 * i + l32) * LROW + 16 * kc + 8 * half]);
            bf[i] = *reinterpret_cast<const bf16x8_t *>(
                &Bs[(buf * BN + wn * 128 + 32 * i + l32) * LROW + 16 * kc + 8 * half]);
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
        bf16x8_t af[2][4], bf[2][4];
        load_frags(buf, 0, af[0], bf[0]);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            // The next step's fragment reads are issued before this step's
            // products (scheduling barriers keep them there), so their LDS
            // latency hides behind 16 MFMAs.
            if (kc + 1 < KC) load_frags(buf, kc + 1, af[(kc + 1) & 1], bf[(kc + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            // C^T blocks: rows = n (W rows), cols = m (x rows) -> a lane owns one m.
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[kc & 1][j], af[kc & 1][i],
                                                                        acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
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

constexpr size_t kLdsBytes = size_t(2) * (BM + BN) * LROW * 2;

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
    // A 256-row tile of either operand is addressed with 32-bit byte offsets.
    if (int64_t(BM) * hidden * 2 >= (int64_t(1) << 31))
        return fail(VSA_ERR_UNSUPPORTED, "hidden = %d is too large", hidden);
    const int64_t blocks = (rows + BM - 1) / BM * ((out_features + BN - 1) / BN);
    if (blocks > 0x7fffffff) return fail(VSA_ERR_ARG, "too many rows");
    if (int st = check_device()) return st;
    if (rows == 0) return VSA_OK;
    static bool attr_set = false;  // per process: the kernel needs more than 64 KB of LDS
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&gate_gemm_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsBytes)) != hipSuccess)
            return fail(VSA_ERR_DEVICE, "cannot raise the LDS limit of the gate GEMM");
        attr_set = true;
    }
    (void)hipGetLastError();
    {
        KernelTimer t(K_GATE_GEMM, static_cast<hipStream_t>(stream));
        hipLaunchKernelGGL(gate_gemm_kernel, dim3(unsigned(blocks)), dim3(256), kLdsBytes,
                           static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(w_gate), rows, int(out_features), int(hidden),
                           static_cast<uint16_t *>(g));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return VSA_OK;
}
