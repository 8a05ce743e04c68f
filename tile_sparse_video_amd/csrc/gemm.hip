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
// fp32. 64-wide k-slices of both operands alternate between two LDS stages
// (128 KB) filled by buffer-to-LDS loads: the data never passes through VGPRs
// and no LDS store instructions are issued. The loads of slice ks + 1 are
// spread over the first three 16-wide k-steps of slice ks (half, a quarter, a
// quarter), placed one after each product together with the next step's
// fragment reads, so they never hold up the matrix-core issue and have time
// to land before the slice ends. A staged row
// is 128 bytes (eight 16-byte chunks); chunk c of row r sits in slot
// c ^ ((r ^ (r >> 3)) & 7), so that one load instruction still covers eight
// whole rows (coalesced) while the MFMA fragment reads (32 rows, one chunk)
// hit distinct LDS banks. After each slice every wave waits for its own loads
// and a barrier (no fence: the compiler's own waits would hold back the
// loads in flight) publishes the next slice and frees the current stage.
//
// Tile order: workgroups are dispatched to the 8 XCDs round robin (blockIdx %
// 8); each XCD takes a contiguous range of logical tiles, and logical tiles
// run over groups of 8 row blocks, row block fastest, so that the workgroups
// resident on one XCD share x rows and W rows in its L2.
#include <hip/hip_runtime.h>

#include "common.h"
#include "device.h"

namespace vsa {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NS = 2;
constexpr int RB = BK * 2;        // bytes per staged row
constexpr int OPB = BM * RB;      // bytes per operand per stage (32 KB)
constexpr int STAGE = 2 * OPB;    // 64 KB
constexpr size_t kLdsBytes = size_t(NS) * STAGE;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource word 3, 32-bit data (gfx9 family)

// s_waitcnt immediate (gfx9 encoding): at most n vector-memory loads
// outstanding, the export and LDS counters left alone.
#define VSA_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

__device__ __forceinline__ int chunk_slot(int c, int r) { return c ^ ((r ^ (r >> 3)) & 7); }

__global__ __launch_bounds__(256, 1) void gate_gemm_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w, int64_t M,
                                                          int N, int K, uint16_t *__restrict__ g)
{
    extern __shared__ __attribute__((aligned(16))) char ring[];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / 2, wn = wave % 2, l32 = lane & 31, half = lane >> 5;
    const int nblocks = (N + BN - 1) / BN;
    const int total = int(gridDim.x);
    const int b = int(blockIdx.x), x8 = b % 8, per = total / 8, rem = total % 8;
    const int lb = x8 < rem ? x8 * (per + 1) + b / 8 : rem * (per + 1) + (x8 - rem) * per + b / 8;
    const int mrows = int((M + BM - 1) / BM);
    const int grp = lb / (8 * nblocks), gm0 = grp * 8, gsz = min(8, mrows - gm0);
    const int in = lb - grp * 8 * nblocks;
    const int mb = __builtin_amdgcn_readfirstlane(gm0 + in % gsz);
    const int64_t m0 = int64_t(mb) * BM;
    const int n0 = __builtin_amdgcn_readfirstlane(in / gsz) * BN;

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

    // Load j (< 8) of this wave fills rows 8 (8 wave + j) .. +7 of an operand:
    // lane -> row + lane / 8, LDS slot lane % 8 (the instruction writes lane l
    // at its LDS base + 16 l), holding the row's chunk whose slot that is. The
    // slice's k offset goes in the scalar offset. Part p (< 4) of a slice is
    // loads 2p and 2p + 1 of both operands.
    uint32_t voff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = (8 * wave + j) * 8 + lane / 8;
        voff[j] = uint32_t(r) * row_bytes + 16u * uint32_t(chunk_slot(lane % 8, r));
    }
    auto issue = [&](int ks, int stage, int p) {
        char *st = ring + stage * STAGE;
#pragma unroll
        for (int j = 2 * p; j < 2 * p + 2; ++j) {
            const int rbase = (8 * wave + j) * 8 * RB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void *)(st + rbase), 16, voff[j], ks * RB, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void *)(st + OPB + rbase), 16, voff[j], ks * RB, 0, 0);
        }
    };
    // Fragment of k-step kc (< 4) of row block i: row R = 128 w + 32 i + l32,
    // chunk 2 kc + half, slot chunk ^ (l32 & 7) ^ (l32 >> 3) ^ 4 (i & 1).
    const int fl = (l32 & 7) ^ (l32 >> 3);
    const int a_row = (wm * 128 + l32) * RB, b_row = OPB + (wn * 128 + l32) * RB;
    auto load_frags = [&](const char *st, int kc, bf16x8_t (&af)[4], bf16x8_t (&bf)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cs = 16 * ((2 * kc + half) ^ fl ^ (4 * (i & 1)));
            af[i] = *reinterpret_cast<const bf16x8_t *>(st + a_row + 32 * i * RB + cs);
            bf[i] = *reinterpret_cast<const bf16x8_t *>(st + b_row + 32 * i * RB + cs);
        }
    };

    f32x16_t acc[4][4];  // [m block][n block]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    const int nk = K / BK;
#pragma unroll
    for (int p = 0; p < 4; ++p) issue(0, 0, p);
    __builtin_amdgcn_s_waitcnt(VSA_VMCNT(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // slice 0 has landed
    asm volatile("" ::: "memory");
    for (int ks = 0; ks < nk; ++ks) {
        const char *st = ring + (ks % NS) * STAGE;
        bf16x8_t af[2][4], bf[2][4];
        load_frags(st, 0, af[0], bf[0]);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            __builtin_amdgcn_sched_barrier(0);
            if (kc + 1 < 4) load_frags(st, kc + 1, af[(kc + 1) & 1], bf[(kc + 1) & 1]);
            // The next slice's loads go into the stage of slice ks - 1, consumed:
            // parts 0 and 1 in the first k-step, 2 and 3 in the second and third,
            // none in the last, so every part has at least two k-steps to land
            // before the slice's wait (-4.5 % against one part per step). The
            // last slice loads itself again (in bounds, never read): no branch,
            // so the loads can be scheduled among the products.
            const int nks = min(ks + 1, nk - 1), nst = (ks + 1) % NS;
            if (kc == 0) {
                issue(nks, nst, 0);
                issue(nks, nst, 1);
            }
            if (kc == 1) issue(nks, nst, 2);
            if (kc == 2) issue(nks, nst, 3);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[kc & 1][j], af[kc & 1][i],
                                                                        acc[i][j], 0, 0, 0);
            // After each product at most one fragment read and one
            // buffer-to-LDS load, so the matrix core is not left idle while a
            // block of loads issues.
            const int n_vmem = kc == 0 ? 8 : kc < 3 ? 4 : 0;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
                if (kc < 3 && t < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                if (t < n_vmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // global read
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);         // this slice's LDS reads are done
        __builtin_amdgcn_s_waitcnt(VSA_VMCNT(0));   // slice ks + 1 has landed (own loads)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
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

#undef VSA_VMCNT

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
