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

// The k loop of one 256 x 256 tile: acc[i][j] (wave (wm, wn) = (wave / 2,
// wave % 2): rows 128 wm + 32 i, columns 128 wn + 32 j) = A . B^T over K, the
// A rows loaded through ra at byte offsets voff_a and the B rows through rb at
// voff_b (loads outside a resource return zero).
__device__ __forceinline__ void gemm_tile(char *ring, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const uint32_t (&voff_a)[8], const uint32_t (&voff_b)[8], int K,
                                          int wave, int lane, f32x16_t (&acc)[4][4])
{
    const int wm = wave / 2, wn = wave % 2, l32 = lane & 31, half = lane >> 5;
    // Load j (< 8) of this wave fills staged rows 8 (8 wave + j) .. +7 of an
    // operand from the caller's byte offsets (the instruction writes lane l at
    // its LDS base + 16 l); the slice's k offset goes in the scalar offset.
    // Part p (< 4) of a slice is loads 2p and 2p + 1 of both operands.
    auto issue = [&](int ks, int stage, int p) {
        char *st = ring + stage * STAGE;
#pragma unroll
        for (int j = 2 * p; j < 2 * p + 2; ++j) {
            const int rbase = (8 * wave + j) * 8 * RB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void *)(st + rbase), 16, voff_a[j], ks * RB, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void *)(st + OPB + rbase), 16, voff_b[j], ks * RB, 0, 0);
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
}

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
    // lane -> row + lane / 8, LDS slot lane % 8, holding the row's chunk whose
    // slot that is.
    uint32_t voff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = (8 * wave + j) * 8 + lane / 8;
        voff[j] = uint32_t(r) * row_bytes + 16u * uint32_t(chunk_slot(lane % 8, r));
    }
    f32x16_t acc[4][4];  // [m block][n block]
    gemm_tile(ring, ra, rb, voff, voff, K, wave, lane, acc);
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

// ---------------------------------------------------------- chunked producer --
//
// SnackOnAI analysis of ComfyUI-Ref2VA-VSA, "The Code, Annotated", snippet two
// (tile the hidden states before projecting, so the projected tensors come out
// in tile order without further sequence-sized copies) and "Why This Design
// Works" (the chunked QKV producer that avoids a padded full projection).
//
// One GEMM of the layer input, its rows taken in tile order (row r of the
// padded tile order is token row_src[r]; padding rows read as zero), against
// the stacked weights [W_q; W_k; W_v; W_gate] ([4 H D][hidden]). The k loop is
// the gate GEMM's; the epilogue stages the 256 x 256 bf16 tile in LDS and
// writes, per 128-column half (one of q, k, v, g; H D is a multiple of 128):
//   q, g: rows back to natural token order ([S][H D]);
//   k, v: the tile-order MFMA fragments the fine pass reads (the layout the
//         coarse stage's gather writes), padding rows zero;
//   q, k, v: the tile means, one thread per column summing the tile's real
//         rows in ascending order in fp32 and dividing once (the canonical
//         order of the coarse stage).
// Only the rows that exist are projected: padding rows cost MFMA work only for
// the partial tiles (zero inputs) and are never stored.
struct ProducerArgs {
    const uint16_t *x;        // [S][K]
    const uint16_t *w;        // [4 H D][K]
    const int32_t *row_src;   // [S_pad]
    const int32_t *block_len; // [n_t]
    int64_t S;
    int S_pad, K, H, n_t;
    uint16_t *q, *g;          // [S][H D]
    uint16_t *kt, *vt;        // fragments [H][n_t][B/64][D/8][64][8]
    float *qm, *km, *vm;      // [H][n_t][D]
};

// Byte address in the staged 256 x 256 bf16 tile of 16-byte chunk c (< 32) of
// row r: chunks are XOR-swizzled by row so that column reads (all 256 threads on
// one row) and the accumulator writes (32 rows, one chunk) spread over the banks.
__device__ __forceinline__ int tile_chunk(int r, int c) { return r * 512 + ((c ^ (r & 31)) << 4); }

template <int D, int B>
__global__ __launch_bounds__(256, 1) void qkv_gemm_kernel(ProducerArgs a)
{
    constexpr int SUB = B / 64, FR = D / 8;
    extern __shared__ __attribute__((aligned(16))) char ring[];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / 2, wn = wave % 2, l32 = lane & 31, half = lane >> 5;
    const int HD = a.H * D, N = 4 * HD, K = a.K;
    const int64_t M = a.S_pad;
    const int nblocks = N / BN;
    const int total = int(gridDim.x);
    const int b = int(blockIdx.x), x8 = b % 8, per = total / 8, rem = total % 8;
    const int lb = x8 < rem ? x8 * (per + 1) + b / 8 : rem * (per + 1) + (x8 - rem) * per + b / 8;
    const int mrows = int((M + BM - 1) / BM);
    const int grp = lb / (8 * nblocks), gm0 = grp * 8, gsz = min(8, mrows - gm0);
    const int in = lb - grp * 8 * nblocks;
    const int mb = __builtin_amdgcn_readfirstlane(gm0 + in % gsz);
    const int m0 = mb * BM;
    const int n0 = __builtin_amdgcn_readfirstlane(in / gsz) * BN;

    // A rows gathered in tile order through one resource over the whole input;
    // a padding row points past its end, so its loads return zero.
    const uint32_t row_bytes = uint32_t(K) * 2;
    const uint32_t a_bytes = uint32_t(a.S) * row_bytes;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.x, (short)0, a_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.w + int64_t(n0) * K), (short)0, uint32_t(BN) * row_bytes, kRsrcWord3);
    uint32_t voff_a[8], voff_b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = (8 * wave + j) * 8 + lane / 8;
        const int m = m0 + r;
        const int tok = m < a.S_pad ? a.row_src[m] : -1;
        const uint32_t slot = 16u * uint32_t(chunk_slot(lane % 8, r));
        voff_a[j] = tok >= 0 ? uint32_t(tok) * row_bytes + slot : a_bytes;
        voff_b[j] = uint32_t(r) * row_bytes + slot;
    }
    f32x16_t acc[4][4];
    gemm_tile(ring, ra, rb, voff_a, voff_b, K, wave, lane, acc);

    // ---- stage the bf16 tile (the ring is free: gemm_tile ends on a barrier)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 128 + 32 * i + l32;
                const int col = wn * 128 + 32 * j + 8 * r + 4 * half;
                uint2 v;
                v.x = uint32_t(f32_to_bf16(acc[i][j][4 * r + 0])) | (uint32_t(f32_to_bf16(acc[i][j][4 * r + 1])) << 16);
                v.y = uint32_t(f32_to_bf16(acc[i][j][4 * r + 2])) | (uint32_t(f32_to_bf16(acc[i][j][4 * r + 3])) << 16);
                *reinterpret_cast<uint2 *>(ring + tile_chunk(row, col >> 3) + 8 * half) = v;
            }
    __syncthreads();
    auto elem = [&](int row, int col) -> float {
        return bf16_to_f32(*reinterpret_cast<const uint16_t *>(ring + tile_chunk(row, col >> 3) + 2 * (col & 7)));
    };

    // ---- tile means of q, k, v: thread = column, rows of each tile in order
    {
        const int c = tid, n = n0 + c, part = n / HD;
        if (part < 3) {
            const int hd = n % HD, h = hd / D, d = hd % D;
            float *mean = part == 0 ? a.qm : (part == 1 ? a.km : a.vm);
#pragma unroll
            for (int t = 0; t < BM / B; ++t) {
                const int tile = m0 / B + t;
                if (tile >= a.n_t) break;
                const int nr = a.block_len[tile];
                float s = 0.0f;
                for (int r = 0; r < nr; ++r) s = s + elem(t * B + r, c);
                mean[(size_t(h) * a.n_t + tile) * D + d] = s / float(nr);
            }
        }
    }
    // ---- per 128-column half: natural rows (q, g) or fragments (k, v)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int nc = n0 + 128 * hf, part = nc / HD, hd0 = nc % HD;
        if (part == 0 || part == 3) {
            uint16_t *dst = part == 0 ? a.q : a.g;
            for (int idx = tid; idx < BM * 16; idx += 256) {
                const int r = idx / 16, ch = idx % 16, m = m0 + r;
                if (m >= a.S_pad) break;  // rows are taken in order
                const int tok = a.row_src[m];
                if (tok < 0) continue;
                const uint4 v = *reinterpret_cast<const uint4 *>(ring + tile_chunk(r, 16 * hf + ch));
                *reinterpret_cast<uint4 *>(dst + size_t(tok) * HD + hd0 + 8 * ch) = v;
            }
        } else {
            uint16_t *dst = part == 1 ? a.kt : a.vt;
            constexpr int NH = 128 / D;
            for (int idx = tid; idx < (BM / 64) * NH * FR * kWave; idx += 256) {
                const int ln = idx % kWave, f = (idx / kWave) % FR;
                const int hl = (idx / (kWave * FR)) % NH, s64 = idx / (kWave * FR * NH);
                const int row0 = m0 + 64 * s64;
                if (row0 >= a.S_pad) break;
                const int tile = row0 / B, sub = (row0 % B) / 64;
                const int lh = ln / 32, ll = ln % 32;
                const int cbase = 128 * hf + hl * D;
                uint4 v;
                if (part == 1) {
                    // K fragment f = kb (D/16) + c: row 32 kb + l, d = 16 c + 8 half + e
                    const int kb = f / (D / 16), c = f % (D / 16);
                    v = *reinterpret_cast<const uint4 *>(ring + tile_chunk(64 * s64 + 32 * kb + ll, (cbase + 16 * c) / 8 + lh));
                } else {
                    // V fragment f = db 4 + c: d = 32 db + l, rows 16 c + {4 half + e, 8 + 4 half + e}
                    const int db = f / 4, c = f % 4, col = cbase + 32 * db + ll;
                    const int r0 = 64 * s64 + 16 * c + 4 * lh;
                    uint16_t e8[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        e8[e] = *reinterpret_cast<const uint16_t *>(ring + tile_chunk(r0 + e, col >> 3) + 2 * (col & 7));
                        e8[4 + e] = *reinterpret_cast<const uint16_t *>(ring + tile_chunk(r0 + 8 + e, col >> 3) + 2 * (col & 7));
                    }
                    v = *reinterpret_cast<const uint4 *>(e8);
                }
                const int h = hd0 / D + hl;
                const size_t frag = ((size_t(h) * a.n_t + tile) * SUB + sub) * FR + f;
                *reinterpret_cast<uint4 *>(dst + frag * 512 + ln * 8) = v;
            }
        }
    }
}

template <int D, int B>
void launch_qkv(const ProducerArgs &a, hipStream_t st)
{
    const int64_t blocks = (int64_t(a.S_pad) + BM - 1) / BM * (4 * a.H * D / BN);
    KernelTimer t(K_QKV_PROJ, st);
    hipLaunchKernelGGL((qkv_gemm_kernel<D, B>), dim3(unsigned(blocks)), dim3(256), kLdsBytes, st, a);
}

template <int D, int B>
int qkv_lds_attr()
{
    static bool done = false;  // per process: the kernel needs more than 64 KB of LDS
    if (!done) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&qkv_gemm_kernel<D, B>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsBytes)) != hipSuccess)
            return VSA_ERR_DEVICE;
        done = true;
    }
    return VSA_OK;
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

extern "C" int vsa_qkv_gate_proj(const vsa_plan_info *info, const int32_t *row_src_dev,
                                 const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                 int32_t hidden, const void *x, const void *w_qkvg, void *q, void *gate,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    clear_error();
    const char *name = "vsa_qkv_gate_proj";
    if (int st = check_info(info)) return st;
    if (heads <= 0) return fail(VSA_ERR_ARG, "%s: heads = %d", name, heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: head_dim = %d; supported: 64, 128", name, head_dim);
    if (hidden <= 0 || hidden % 64 != 0)
        return fail(VSA_ERR_UNSUPPORTED, "%s: hidden = %d must be a positive multiple of 64", name, hidden);
    if ((int64_t(heads) * head_dim) % 128 != 0)
        return fail(VSA_ERR_UNSUPPORTED, "%s: heads x head_dim = %lld must be a multiple of 128", name,
                    (long long)heads * head_dim);
    if (!row_src_dev || !block_len_dev || !x || !w_qkvg || !q || !gate || !workspace)
        return fail(VSA_ERR_ARG, "%s: null device pointer", name);
    // The input rows are addressed with 32-bit byte offsets (plus one slice past the end).
    if ((info->rows_real + 1) * int64_t(hidden) * 2 >= (int64_t(1) << 32) ||
        int64_t(BM) * hidden * 2 >= (int64_t(1) << 31))
        return fail(VSA_ERR_UNSUPPORTED, "%s: %lld tokens x hidden %d exceed 4 GiB of input", name,
                    (long long)info->rows_real, hidden);
    vsa_ws_layout L;
    compute_layout(*info, heads, head_dim, 1, &L);
    if (workspace_bytes < L.part_o)
        return fail(VSA_ERR_ARG, "%s: workspace has %zu bytes, needs %zu", name, workspace_bytes, L.part_o);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(VSA_ERR_ARG, "%s: workspace must be 256-byte aligned", name);
    if (int st = check_device()) return st;
    char *ws = static_cast<char *>(workspace);
    ProducerArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint16_t *>(w_qkvg);
    a.row_src = row_src_dev;
    a.block_len = block_len_dev;
    a.S = info->rows_real;
    a.S_pad = int(info->rows_padded);
    a.K = hidden;
    a.H = heads;
    a.n_t = info->n_tiles;
    a.q = static_cast<uint16_t *>(q);
    a.g = static_cast<uint16_t *>(gate);
    a.kt = reinterpret_cast<uint16_t *>(ws + L.k_tiled);
    a.vt = reinterpret_cast<uint16_t *>(ws + L.v_tiled);
    a.qm = reinterpret_cast<float *>(ws + L.q_mean);
    a.km = reinterpret_cast<float *>(ws + L.k_mean);
    a.vm = reinterpret_cast<float *>(ws + L.v_mean);
    const int B = info->tile_rows;
    const int attr = head_dim == 128 ? (B == 64 ? qkv_lds_attr<128, 64>() : qkv_lds_attr<128, 128>())
                                     : (B == 64 ? qkv_lds_attr<64, 64>() : qkv_lds_attr<64, 128>());
    if (attr != VSA_OK) return fail(VSA_ERR_DEVICE, "%s: cannot raise the LDS limit", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (head_dim == 128) {
        if (B == 64) launch_qkv<128, 64>(a, st);
        else launch_qkv<128, 128>(a, st);
    } else {
        if (B == 64) launch_qkv<64, 64>(a, st);
        else launch_qkv<64, 128>(a, st);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    return VSA_OK;
}
