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
//    query rows for its whole key list, so the K/V of a key tile is consumed
//    by exactly one wave and never has to be shared through LDS: K and V arrive
//    as fully coalesced 1 KB fragments (the layout the coarse stage writes)
//    straight into VGPRs through bounds-checked buffer loads.
//  - S^T = K . Q^T and O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 with fp32
//    accumulation. With keys as rows of S^T, each lane owns one query column,
//    so the running max / sum and the O rescale are per lane (plus one
//    cross-half exchange), and the S accumulator already has the register
//    layout of the P^T operand of the second product.
//  - The key list is walked in 32-key halves; K of the next half is fetched
//    once both S products are issued and V once P.V is issued. 256 VGPRs per
//    wave give two waves per SIMD, which cover each other's memory waits. The
//    bf16 step is scheduled by hand so that each query block's softmax runs
//    on the vector unit while the matrix core works on the other block's
//    products (scheduling barriers pin the interleaving); the kernel is
//    power-limited, so the gain is small (1-5 %) but free.
//  - With random keep-sets the kernel is bound by the traffic beyond L2, so
//    for large heads the key list is split into C chunks by tile id modulo C,
//    and chunk c is dispatched to XCD c (workgroups are spread round-robin
//    over the 8 XCDs): each XCD's L2 then serves only 1/C of a head's K/V,
//    swept in ascending order by all its waves. Each chunk writes a partial
//    (O / l in bf16, running max and sum in fp32); a merge kernel combines the
//    chunks and applies the gated epilogue. Small heads (C = 1) finish in the
//    epilogue. Heads too large for the Infinity Cache use 8 * G chunks, taken
//    in G phases per head.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "device.h"

namespace vsa {

// Number of key chunks for the fine pass. Split (8 chunks, one per XCD) when
// the K and V of one head are large enough that L2 reuse across query tiles
// matters; beyond 96 MiB per head use 8 * G chunks taken in G phases, so the
// K/V touched by one phase stays within what the Infinity Cache serves at
// full speed. With 64-row tiles and more than 32 MiB per head (an eighth of
// the head no longer fits one XCD's 4 MB L2) take at least two phases: at the
// H3-shaped layer 16 chunks make fine + merge 2.3 % faster than 8. 128-row
// tiles keep 8: their key lists are short (the Veda-style layer keeps 114
// tiles), and 16 chunks made it 9 % slower.
int auto_split_chunks(const vsa_plan_info &info, int head_dim)
{
    const double mib = 1024.0 * 1024.0;
    const double head_kv = 2.0 * double(info.rows_padded) * head_dim * 2.0;
    if (head_kv < 16.0 * mib) return 1;
    int phases = int(std::ceil(head_kv / (96.0 * mib)));
    if (info.tile_rows == 64 && head_kv > 32.0 * mib) phases = std::max(phases, 2);
    return 8 * std::min(phases, 8);
}

int resolve_split(const vsa_plan_info &info, int head_dim, int32_t requested, int *chunks)
{
    if (requested < 0 || requested > kMaxSplit)
        return fail(VSA_ERR_ARG, "split_chunks = %d outside [0, %d] (0 = automatic)", requested, kMaxSplit);
    *chunks = requested > 0 ? requested : auto_split_chunks(info, head_dim);
    return VSA_OK;
}

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
    uint16_t *part_o;           // split: [items][C][DB][2][2][64][8] bf16 O / l
    float *part_ml;             // split: [items][C][2 (m, l)][2][32]
    int H, P, n_v, n_t, k, chunks;
    int ld;                     // heads per token row of q, gate, out and dout (>= H)
    int ref;                    // reference sparsity: every tile has an explicit list
    int list_len;               // ref: entries per list (k_ref + k_gen), keep is [H][n_t][list_len]
    // Statistics merge (backward support): per tile-order row, the log2-domain
    // log-sum-exp and D_t = dout . O_fine instead of the gated output.
    const uint16_t *dout;       // [S][H][D]
    float *lse_out, *dt_out;    // [H][S_pad]
    // Training forward: the gated output plus, per tile-order row, the lse and
    // the normalised fine output O_fine in fp32 ([H][S_pad][D]).
    float *ofine_out;
    // INT8 scores: K codes in tile order [H][n_t][B/64][2][D/32][64][16] and one
    // scale per 64-row block [H][n_t][B/64].
    const uint8_t *k8;
    const float *k_scale;
    float scale_log2e;
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t load_frag(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8_t *>(p);
}

constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr float kLazy = 8.0f;   // log2-domain slack before the running max moves
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource word 3, 32-bit data (gfx9 family)
constexpr int kListCap = 896;   // key-list entries staged in LDS per segment
constexpr int kFillBatch = 4;   // 64-position blocks of the key list read per round

// Max / sum of a value and its copy in the lane 32 apart (same query column of
// the other row half): v_permlane32_swap exchanges the upper half of one
// register with the lower half of another, so both halves see both values in
// the same order and agree bit for bit.
__device__ __forceinline__ float xhalf_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Gated epilogue of the query row that this lane holds in column qb of O^T
// (element 4i + j of O[db][qb] <-> d = 32db + 8i + 4half + j):
// out[base + d] = bf16(O[d] * inv + g[base + d] * oc[d]). Every gate and
// O_coarse load is issued before the first store (the compiler cannot move a
// load across a store to memory it cannot prove distinct), so the row's loads
// are in flight together.
template <int DB, typename OArr>
__device__ __forceinline__ void gated_row(uint16_t *out, const uint16_t *gate, size_t base,
                                          const float *oc, const OArr &O, int qb, float inv, int half)
{
    uint2 graw[DB][4];
    float4 ocv[DB][4];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            graw[db][i] = *reinterpret_cast<const uint2 *>(gate + base + d0);
            ocv[db][i] = *reinterpret_cast<const float4 *>(oc + d0);
        }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            const uint2 g = graw[db][i];
            const float4 c = ocv[db][i];
            const float o0 = O[db][qb][4 * i], o1 = O[db][qb][4 * i + 1];
            const float o2 = O[db][qb][4 * i + 2], o3 = O[db][qb][4 * i + 3];
            const bf16x2_t w0 = {(__bf16)(o0 * inv + __uint_as_float(g.x << 16) * c.x),
                                 (__bf16)(o1 * inv + __uint_as_float(g.x & 0xffff0000u) * c.y)};
            const bf16x2_t w1 = {(__bf16)(o2 * inv + __uint_as_float(g.y << 16) * c.z),
                                 (__bf16)(o3 * inv + __uint_as_float(g.y & 0xffff0000u) * c.w)};
            uint2 w;
            w.x = __builtin_bit_cast(uint32_t, w0);
            w.y = __builtin_bit_cast(uint32_t, w1);
            *reinterpret_cast<uint2 *>(out + base + d0) = w;
        }
}

template <int D, int B, bool SPLIT, bool I8 = false>
__global__ __launch_bounds__(64, 2) void fine_attn_kernel(FineArgs a)
{
    constexpr int SUB = B / 64;   // 64-row blocks per tile
    constexpr int NC = D / 16;    // reduction chunks of S = K.Q^T
    constexpr int NC8 = D / 32;   // INT8: reduction chunks of 32 codes
    constexpr int KN = I8 ? NC8 : NC;  // K registers (16 bytes each) per 32-key half
    constexpr int DB = D / 32;    // 32-row blocks of O^T (over d)
    constexpr int FR = D / 8;     // 1 KB fragments per 64-row block
    constexpr int HPU = 2 * SUB;  // 32-key halves per key tile
    const int lane = threadIdx.x;
    const int l32 = lane & 31, half = lane >> 5;

    // ---- work item, head-major so the K/V in flight belong to one or two heads.
    // Split: the chunk's low three bits are block % 8, so chunk c always runs on
    // XCD c % 8; with C = 8G the G phases of a head run one after another.
    const int per_head = a.n_t * SUB;
    int item, chunk = 0;
    if (!SPLIT) {
        item = blockIdx.x;  // = (h * n_t + tile) * SUB + qsub
    } else if (a.chunks % 8 == 0) {
        const int G = a.chunks / 8, rest = blockIdx.x / 8;
        const int hh = rest / (G * per_head), g = (rest / per_head) % G;
        item = hh * per_head + rest % per_head;
        chunk = 8 * g + blockIdx.x % 8;
    } else {
        item = blockIdx.x / a.chunks;
        chunk = blockIdx.x % a.chunks;
    }
    const int h = item / per_head;
    const int r = item % per_head;
    const int tile = r / SUB, qsub = r % SUB;
    const bool dense = !a.ref && tile < a.P;
    const int n_list = a.ref ? a.list_len : dense ? a.n_t : a.P + a.k;

    // ---- query fragments (B operand of S^T = K . Q^T): lane -> query 32qb + l32,
    // reduction slot e of chunk c -> d = 16c + 8*half + e. Staged once in LDS
    // (16 KB per wave) and re-read for every S product.
    __shared__ __attribute__((aligned(16))) bf16x8_t q_lds[2][NC][kWave];
    __shared__ uint32_t list_lds[kListCap];  // tile | (block_len - 1) << 25
    __shared__ float list_sk[I8 ? kListCap * SUB : 1];  // INT8: K block scales of the entries
    int tok[2];
    float sq = 0.f;  // INT8: the scale of this 64-row query block
    if constexpr (!I8) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) tok[qb] = a.row_src[size_t(tile) * B + 64 * qsub + 32 * qb + l32];
        // The block's 64 Q rows, D / 8 lanes per row (16 bytes each, so a load
        // covers whole rows), then stored to their fragment slots: piece p of
        // row r is chunk p / 2, slot half p % 2, column r % 32 of block r / 32.
        constexpr int PPR = D / 8, RPI = kWave / PPR, NG = 64 / RPI;
        const int pr = lane / PPR, pp = lane % PPR;
        bf16x8_t qv[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int tk = a.row_src[size_t(tile) * B + 64 * qsub + RPI * g + pr];
            const bf16x8_t v = load_frag(a.q + (size_t(tk < 0 ? 0 : tk) * a.ld + h) * D + 8 * pp);
            qv[g] = tk < 0 ? bf16x8_t{} : v;
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int r = RPI * g + pr;
            q_lds[r >> 5][pp >> 1][(pp & 1) * 32 + (r & 31)] = qv[g];
        }
    } else {
        // INT8 B operand: lane -> query 32qb + l32, code slot e of chunk c ->
        // d = 32c + 16*half + e (the K codes use the same slots). The block's
        // scale is max|q| / 127 over its 64 rows (padding rows are zero); the
        // codes are round-half-even(q * (127 / max|q|)), all in fp32.
        u32x4_t raw[2][NC8][2];
        float amax = 0.f;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            tok[qb] = a.row_src[size_t(tile) * B + 64 * qsub + 32 * qb + l32];
            const uint16_t *qrow = a.q + (size_t(tok[qb] < 0 ? 0 : tok[qb]) * a.ld + h) * D + 16 * half;
#pragma unroll
            for (int c = 0; c < NC8; ++c)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    u32x4_t v = *reinterpret_cast<const u32x4_t *>(qrow + 32 * c + 8 * j);
                    if (tok[qb] < 0) v = u32x4_t{};
                    raw[qb][c][j] = v;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[w] << 16)),
                                                 fabsf(__uint_as_float(v[w] & 0xffff0000u))));
                }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        amax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(amax)));
        const float inv = amax > 0.f ? 127.0f / amax : 0.f;
        sq = amax > 0.f ? amax / 127.0f : 0.f;
        auto code = [&](float x) -> uint32_t {
            const float y = fminf(fmaxf(__builtin_rintf(x * inv), -127.f), 127.f);
            return uint32_t(int(y)) & 0xffu;
        };
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int c = 0; c < NC8; ++c) {
                u32x4_t w;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const uint32_t r0 = raw[qb][c][j][2 * t2], r1 = raw[qb][c][j][2 * t2 + 1];
                        w[2 * j + t2] = code(__uint_as_float(r0 << 16)) |
                                        code(__uint_as_float(r0 & 0xffff0000u)) << 8 |
                                        code(__uint_as_float(r1 << 16)) << 16 |
                                        code(__uint_as_float(r1 & 0xffff0000u)) << 24;
                    }
                q_lds[qb][c][lane] = as_bf16x8(w);
            }
    }

    // ---- key list source. Default: position n -> tile n (prefix, or all tiles
    // for a dense query tile) or the n-P-th kept tile. Reference sparsity: the
    // n-th entry of the tile's own list. Entries are clamped (this only guards
    // against a foreign list).
    const int32_t *keep_row = a.ref ? a.keep + (size_t(h) * a.n_t + tile) * a.list_len
                              : dense ? a.keep
                                      : a.keep + (size_t(h) * a.n_v + (tile - a.P)) * a.k;
    // Tiles of list positions n (0 <= n < n_list). The list loads are issued for
    // every lane (at clamped positions) whenever the wave's list has stored
    // entries, all in one block, and the values are chosen afterwards, so no
    // load sits behind a per-lane branch or waits for another.
    const bool from_keep = a.ref || (!dense && a.k > 0);  // wave-uniform
    auto tiles_at = [&](const int (&n)[kFillBatch], int (&t)[kFillBatch]) {
        int kv[kFillBatch];
#pragma unroll
        for (int u = 0; u < kFillBatch; ++u) kv[u] = 0;
        if (from_keep) {
#pragma unroll
            for (int u = 0; u < kFillBatch; ++u)
                kv[u] = keep_row[a.ref ? min(n[u], a.list_len - 1) : min(max(n[u] - a.P, 0), a.k - 1)];
        }
#pragma unroll
        for (int u = 0; u < kFillBatch; ++u) {
            const int c = min(max(kv[u], 0), a.n_t - 1);
            t[u] = a.ref ? c : ((dense || n[u] < a.P) ? n[u] : c);
        }
    };
    // The wave stages the next segment of its key list (tiles of this chunk)
    // into LDS with block_len packed alongside. Four blocks of 64 list
    // positions are read per round: their entries, then their tiles' block
    // lengths (and INT8 block scales), each batch in flight together.
    int scan = 0;
    auto fill = [&]() -> int {
        int count = 0;
        bool full = false;
        while (!full && scan < n_list) {
            int pos[kFillBatch], tt[kFillBatch], bl[kFillBatch];
            float sk[I8 ? kFillBatch * SUB : 1];
#pragma unroll
            for (int u = 0; u < kFillBatch; ++u) pos[u] = min(scan + kWave * u + lane, n_list - 1);
            tiles_at(pos, tt);
#pragma unroll
            for (int u = 0; u < kFillBatch; ++u) {
                bl[u] = a.block_len[tt[u]];
                if constexpr (I8) {
#pragma unroll
                    for (int sb = 0; sb < SUB; ++sb)
                        sk[u * SUB + sb] = a.k_scale[(size_t(h) * a.n_t + tt[u]) * SUB + sb];
                }
            }
#pragma unroll
            for (int u = 0; u < kFillBatch; ++u) {
                if (full || scan >= n_list) break;  // uniform
                const int n = scan + lane, t = tt[u];
                const bool match = n < n_list && (!SPLIT || t % a.chunks == chunk);
                const uint64_t mask = __ballot(match);
                const int take = __popcll(mask);
                if (count + take > kListCap) {  // next segment
                    full = true;
                    break;
                }
                if (match) {
                    const int at = count + __popcll(mask & lanes_below(lane));
                    list_lds[at] = uint32_t(t) | uint32_t(bl[u] - 1) << 25;
                    if constexpr (I8) {
#pragma unroll
                        for (int sb = 0; sb < SUB; ++sb) list_sk[at * SUB + sb] = sk[u * SUB + sb];
                    }
                }
                count += take;
                scan += kWave;
            }
        }
        __syncthreads();
        return count;
    };

    // ---- K/V stream: one buffer resource per head (SGPRs); a fragment is read
    // with an SGPR byte offset plus the lane's 16-byte slot, fully coalesced.
    // Reads outside the head's region return zero instead of faulting.
    const uint32_t head_bytes = uint32_t(a.n_t) * B * D * 2;
    const size_t head_elems = size_t(h) * a.n_t * B * D;
    const __amdgpu_buffer_rsrc_t rk = I8
        ? __builtin_amdgcn_make_buffer_rsrc((void *)(a.k8 + head_elems), (short)0, head_bytes / 2, kRsrcWord3)
        : __builtin_amdgcn_make_buffer_rsrc((void *)(a.kt + head_elems), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void *)(a.vt + head_elems), (short)0, head_bytes, kRsrcWord3);
    const int vlane = lane * 16;
    auto entry = [&](int v) -> uint32_t {  // wave-uniform LDS read
        return __builtin_amdgcn_readfirstlane(list_lds[v / HPU]);
    };
    // Half v covers rows 32*(v % 2) .. +31 of 64-row block (v % HPU) / 2 of its tile.
    auto half_base = [&](int v, uint32_t e) -> uint32_t {  // e = entry(v)
        const uint32_t t = e & 0x1ffffffu;
        return (t * SUB + uint32_t((v % HPU) >> 1)) * FR * 1024u;
    };
    // INT8 codes: a 64-row block is 2 * D/32 fragments of 1 KB (half the bf16 size).
    auto load_k = [&](int v, uint32_t e, u32x4_t (&Kb)[KN]) {
        const uint32_t base = (I8 ? half_base(v, e) / 2 : half_base(v, e)) + uint32_t(v & 1) * KN * 1024u;
#pragma unroll
        for (int c = 0; c < KN; ++c) Kb[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, vlane, base + c * 1024u, 0);
    };
    auto load_v = [&](int v, uint32_t e, u32x4_t (&Vb)[2 * DB]) {
        const uint32_t base = half_base(v, e) + uint32_t(v & 1) * 2 * 1024u;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                Vb[2 * db + cc] = __builtin_amdgcn_raw_buffer_load_b128(rv, vlane, base + (4 * db + cc) * 1024u, 0);
    };

    f32x16_t O[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db][0] = O[db][1] = f32x16_t{};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    const float c2 = a.scale_log2e;
    // Per query block: -m c2 (the exponent offset) and the raw score above
    // which the running max must move (m + kLazy / c2); both change only on a
    // rescale. With m = -inf every finite score moves it.
    float moff[2] = {0.f, 0.f}, thr[2] = {-INFINITY, -INFINITY};

    // One 32-key half of the INT8 pass (the bf16 pass uses step_b below): S =
    // K.Q^T, online softmax, O += V.P. K of the next half is fetched as soon as
    // S is formed, V of the next half once P.V has been issued. The body is straight-line on purpose: halves with no real key are
    // masked rather than skipped, and the last refill re-reads a valid half, so
    // the K/V registers never merge values from different control paths.
    auto step = [&](int v, int n_half, uint32_t ecur, u32x4_t (&Kb)[KN], u32x4_t (&Vb)[2 * DB]) -> uint32_t {
        const int real = min(32, int(ecur >> 25) + 1 - 32 * (v % HPU));
        const int next = v + 1 < n_half ? v + 1 : v;
        // The next half's list entry is read here and handed to the next step,
        // so no step opens with an LDS round trip before its Q reads (-1.5 %).
        const uint32_t enext = entry(next);
        // INT8: score = (integer product) * qk with qk = s_q * s_k of the two
        // blocks; the exponent folds qk into c2. Clamping qk and c2 * qk to the
        // least normal keeps masked keys at -inf (an all-zero block gives
        // integer products of 0, so its scores stay exactly 0).
        float qk = 1.f, c2s = c2;
        if constexpr (I8) {
            const float sk = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(list_sk[v >> 1])));
            qk = fmaxf(sq * sk, 1.17549435e-38f);
            c2s = fmaxf(c2 * qk, 1.17549435e-38f);
        }

        // The two 32-query blocks are independent (each lane owns one query of
        // each), so each block runs S, softmax and P.V on its own: only its S
        // and P are live, and block 1's products can overlap block 0's softmax.
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            // S^T: rows = keys 8i + 4*half + j of this half (acc 4i + j), col = query.
            // Q fragments come from LDS in one batch; the empty asm makes the lane
            // index opaque so they are re-read rather than hoisted into VGPRs.
            int ql = lane;
            asm volatile("" : "+v"(ql));
            f32x16_t S;
            if constexpr (!I8) {
                bf16x8_t Qf[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) Qf[c] = q_lds[qb][c][ql];
                S = f32x16_t{};
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Kb[c]), Qf[c], S, 0, 0, 0);
            } else {
                i32x4_t Qf[NC8];
#pragma unroll
                for (int c = 0; c < NC8; ++c) Qf[c] = __builtin_bit_cast(i32x4_t, q_lds[qb][c][ql]);
                i32x16_t Si = i32x16_t{};
#pragma unroll
                for (int c = 0; c < NC8; ++c)
                    Si = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, Kb[c]), Qf[c], Si, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e) S[e] = float(Si[e]);
            }
            if (qb == 1) load_k(next, enext, Kb);
            // Padding keys (partial tiles only: a wave-uniform branch) never score.
            if (__builtin_expect(real < 32, 0)) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (8 * i + 4 * half + j >= real) S[4 * i + j] = -INFINITY;
            }

            // Online softmax per query column, rescaling lazily: the running max
            // m only moves (and O, l are rescaled) when some row's new max exceeds
            // it by more than kLazy in log2 units, so p <= 2^kLazy stays safe in
            // fp32 and bf16 while most halves skip the rescale entirely.
            // Max over the lane's 16 keys as a v_max3 tree (7 ops instead of 15).
            float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);
#pragma unroll
            for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, S[e]), S[e + 1]);
            mx = fmaxf(mx, S[15]);
            mx = xhalf_max(mx);
            if constexpr (I8) mx *= qk;  // integer units -> score units (qk > 0)
            if (__ballot(mx > thr[qb]) != 0) {
                const float m_new = fmaxf(m[qb], mx);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m[qb] - m_new) * c2);
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) O[db][qb][e] *= alpha;
                m[qb] = m_new;
                moff[qb] = m_new == -INFINITY ? 0.f : -m_new * c2;
                thr[qb] = m_new == -INFINITY ? -INFINITY : m_new + kLazy / c2;
            }
            float rs = 0.f;
            bf16x8_t Pf[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * cc + e], c2s, moff[qb]));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * cc + e + 1], c2s, moff[qb]));
                    const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
                    rs = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, rs, false);
                    w[e / 2] = __builtin_bit_cast(uint32_t, pp);
                }
                // 16-key chunk cc of this half = acc elements 8cc .. 8cc + 7
                Pf[cc] = as_bf16x8(w);
            }
            l[qb] += rs;

            // O^T[db][qb] += V^T[db] . P^T[qb] over the half's two 16-key chunks.
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                f32x16_t acc = O[db][qb];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Vb[2 * db + cc]), Pf[cc], acc, 0, 0, 0);
                O[db][qb] = acc;
            }
        }
        load_v(next, enext, Vb);
        return enext;
    };

    // ---- bf16 step, scheduled by hand. Per 32-key half the matrix core runs
    // 32 products (S of query blocks 0 and 1, then P.V of both) and the vector
    // unit two softmaxes; in program order each softmax is spread over the
    // products it does not depend on (scheduling barriers pin the order):
    //   S0 (8)  |  S1 0-1 + max of S0  |  [rescale O0]  |  S1 2-7 + exp of S0
    //   | P.V0 0-1 + max of S1  |  [rescale O1]  |  P.V0 2-7 + exp of S1  |  P.V1 (8)
    // Q fragments are read from LDS two products ahead.
    // The lane index goes through an empty asm once per step, so the Q reads
    // are re-issued every step (not hoisted into registers) from one base.
    const bf16x8_t *qbase = nullptr;
    auto qread = [&](int qb, int c) -> bf16x8_t { return qbase[(qb * NC + c) * kWave]; };
    // Each lane keeps the max and sum of its own 16 keys of a half: the lazy
    // threshold test is a ballot over all lanes, so the exchange with the other
    // row half (xhalf_max) is needed only when a rescale happens, and the two
    // halves' sums are added once, after the key list.
    auto row_max = [&](const f32x16_t &S) -> float {
        float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, S[e]), S[e + 1]);
        mx = fmaxf(mx, S[15]);
        return mx;
    };
    auto rescale = [&](float mx, int qb) {
        if (__ballot(mx > thr[qb]) != 0) {
            const float m_new = fmaxf(m[qb], xhalf_max(mx));
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m[qb] - m_new) * c2);
            l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) O[db][qb][e] *= alpha;
            m[qb] = m_new;
            moff[qb] = m_new == -INFINITY ? 0.f : -m_new * c2;
            thr[qb] = m_new == -INFINITY ? -INFINITY : m_new + kLazy / c2;
        }
    };
    // Probabilities of elements 2p, 2p + 1 of S (16-key chunk p / 4), packed to
    // bf16 into w[p / 4] and added to the row sum in the same bf16 values.
    auto prob_pair = [&](const f32x16_t &S, int qb, int p, float &rs, u32x4_t (&w)[2]) {
        const int cc = p >> 2, e = 2 * (p & 3);
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * cc + e], c2, moff[qb]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * cc + e + 1], c2, moff[qb]));
        const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
        rs = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, rs, false);
        w[cc][e / 2] = __builtin_bit_cast(uint32_t, pp);
    };
    auto mask_pad = [&](f32x16_t &S, int real) {
        const int lim = real - 4 * half;  // key 8i + 4 half + j is padding iff 8i + j >= lim
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (8 * i + j >= lim) S[4 * i + j] = -INFINITY;
    };
    // pairs of softmax elements placed after product slot i of a 6-slot region
    constexpr int kPairsAt[6] = {2, 2, 1, 1, 1, 1};
    auto step_b = [&](int v, int n_half, uint32_t ecur, u32x4_t (&Kb)[KN], u32x4_t (&Vb)[2 * DB]) -> uint32_t {
        const int real = min(32, int(ecur >> 25) + 1 - 32 * (v % HPU));
        const int next = v + 1 < n_half ? v + 1 : v;
        const uint32_t enext = entry(next);
        {
            int ql = lane;
            asm volatile("" : "+v"(ql));
            qbase = &q_lds[0][0][ql];
        }
        // ---- S0, with the first Q fragments of block 1 read at its end
        bf16x8_t qa = qread(0, 0), qb_ = qread(0, 1), qc;
        f32x16_t S0 = f32x16_t{}, S1 = f32x16_t{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qc = c + 2 < NC ? qread(0, c + 2) : qread(1, c + 2 - NC);
            S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Kb[c]), qa, S0, 0, 0, 0);
            qa = qb_;
            qb_ = qc;
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- S1 products 0-1 with the max of S0
        qc = qread(1, 2);
        S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Kb[0]), qa, S1, 0, 0, 0);
        qa = qb_;
        qb_ = qc;
        qc = qread(1, 3);
        S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Kb[1]), qa, S1, 0, 0, 0);
        qa = qb_;
        qb_ = qc;
        if (__builtin_expect(real < 32, 0)) mask_pad(S0, real);
        const float mx0 = row_max(S0);
        rescale(mx0, 0);
        // ---- S1 products 2-7 with the exponentials of S0
        float rs0 = 0.f;
        u32x4_t w0[2];
        {
            int p = 0;
#pragma unroll
            for (int c = 2; c < NC; ++c) {
                if (c + 2 < NC) qc = qread(1, c + 2);
                S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Kb[c]), qa, S1, 0, 0, 0);
                qa = qb_;
                qb_ = qc;
                const int np = NC == 8 ? kPairsAt[c - 2] : (c + 1 < NC ? 8 / (NC - 2) : 8 - (8 / (NC - 2)) * (NC - 3));
#pragma unroll
                for (int u = 0; u < np; ++u, ++p) prob_pair(S0, 0, p, rs0, w0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        l[0] += rs0;
        const bf16x8_t P0[2] = {as_bf16x8(w0[0]), as_bf16x8(w0[1])};
        load_k(next, enext, Kb);
        __builtin_amdgcn_sched_barrier(0);
        // ---- P.V0 products 0-1 with the max of S1
        O[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Vb[0]), P0[0], O[0][0], 0, 0, 0);
        O[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Vb[1]), P0[1], O[0][0], 0, 0, 0);
        if (__builtin_expect(real < 32, 0)) mask_pad(S1, real);
        const float mx1 = row_max(S1);
        rescale(mx1, 1);
        // ---- P.V0 products 2-7 with the exponentials of S1
        float rs1 = 0.f;
        u32x4_t w1[2];
        {
            int p = 0;
#pragma unroll
            for (int i = 2; i < 2 * DB; ++i) {
                const int db = i >> 1, cc = i & 1;
                O[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Vb[2 * db + cc]), P0[cc], O[db][0], 0, 0, 0);
                const int np = 2 * DB == 8 ? kPairsAt[i - 2] : (i + 1 < 2 * DB ? 8 / (2 * DB - 2) : 8 - (8 / (2 * DB - 2)) * (2 * DB - 3));
#pragma unroll
                for (int u = 0; u < np; ++u, ++p) prob_pair(S1, 1, p, rs1, w1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        l[1] += rs1;
        const bf16x8_t P1[2] = {as_bf16x8(w1[0]), as_bf16x8(w1[1])};
        // ---- P.V1
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                O[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Vb[2 * db + cc]), P1[cc], O[db][1], 0, 0, 0);
        load_v(next, enext, Vb);
        return enext;
    };

    u32x4_t Kb[KN], Vb[2 * DB];
    while (true) {
        const int count = fill();
        if (count > 0) {
            const int n_half = count * HPU;
            uint32_t e = entry(0);
            load_k(0, e, Kb);
            load_v(0, e, Vb);
            for (int v = 0; v < n_half; ++v) {
                if constexpr (I8) e = step(v, n_half, e, Kb, Vb);
                else e = step_b(v, n_half, e, Kb, Vb);
            }
        }
        if (scan >= n_list) break;
        __syncthreads();  // every lane has read the list before it is refilled
    }
    // Each lane summed its own row half: the query's l is the sum of the two.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) l[qb] = xhalf_sum(l[qb]);

    if (SPLIT) {
        // ---- partial: O / l in bf16 (register order), plus fp32 (m, l) per query.
        const size_t pidx = size_t(item) * a.chunks + chunk;
        uint16_t *po = a.part_o + pidx * (64 * D);
        float inv[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) inv[qb] = l[qb] > 0.f ? 1.0f / l[qb] : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                u32x4_t w[2];
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const bf16x2_t pp = {(__bf16)(O[db][qb][e] * inv[qb]), (__bf16)(O[db][qb][e + 1] * inv[qb])};
                    w[e / 8][(e % 8) / 2] = __builtin_bit_cast(uint32_t, pp);
                }
                // Each 16-byte half of the lane's 32 bytes goes to its own 1 KB run
                // (lane-contiguous stores and, in the merge, loads). The partials
                // are read only by the merge: non-temporal stores keep them from
                // displacing the K/V tiles the other waves reuse from L2 (1.5 %
                // faster at the H3-shaped layer, 1.7 % at the long-video one).
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8)
                    __builtin_nontemporal_store(
                        w[h8], reinterpret_cast<u32x4_t *>(po + (((db * 2 + qb) * 2 + h8) * 64 + lane) * 8));
            }
        if (lane < 32) {
            float *pml = a.part_ml + pidx * 128;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                __builtin_nontemporal_store(m[qb], pml + qb * 32 + lane);
                __builtin_nontemporal_store(l[qb], pml + 64 + qb * 32 + lane);
            }
        }
        return;
    }

    // ---- epilogue: out = bf16(O_fine + g * O_coarse[tile]), natural token order.
    // O^T[db][qb] acc 4i + j <-> d = 32db + 8i + 4*half + j, query column l32.
    const float *oc = a.o_coarse + (size_t(h) * a.n_t + tile) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if (tok[qb] < 0) continue;
        const float inv = 1.0f / l[qb];
        gated_row<DB>(a.out, a.gate, (size_t(tok[qb]) * a.ld + h) * D, oc, O, qb, inv, half);
    }
}

// Combines the C chunk partials of one (head, 64 query rows) item:
// M = max_c m_c, w_c = l_c 2^((m_c - M) scale log2 e), O = sum_c w_c (O/l)_c,
// L = sum_c w_c, then the same gated epilogue as the direct path.
// One wavefront per item, lanes laid out as in the fine kernel.
// MODE: kMergeOut = the gated output; kMergeStats = per-row lse and
// D_t = dout . O_fine instead (backward support); kMergeTrain = the gated
// output plus per-row lse and O_fine (a training forward).
constexpr int kMergeOut = 0, kMergeStats = 1, kMergeTrain = 2;
template <int D, int B, int MODE>
__global__ __launch_bounds__(256) void merge_kernel(FineArgs a, int n_items)
{
    constexpr int SUB = B / 64, DB = D / 32;
    const int lane = threadIdx.x % kWave;
    // Waves are numbered tile-major (the heads of one 64-row block side by
    // side), so neighbouring waves read and write adjacent slices of the same
    // token records of g and out (1.7 % faster than head-major at 42 heads).
    const int wi = blockIdx.x * 4 + threadIdx.x / kWave;
    if (wi >= n_items) return;
    const int l32 = lane & 31, half = lane >> 5;
    const int h = wi % a.H;
    const int r = wi / a.H;
    const int item = h * (a.n_t * SUB) + r;
    const int tile = r / SUB, qsub = r % SUB;
    const float c2 = a.scale_log2e;
    const int C = a.chunks;
    const size_t p0 = size_t(item) * C;
    int tok[2];  // the rows' tokens (-1: padding), read up front
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) tok[qb] = a.row_src[size_t(tile) * B + 64 * qsub + 32 * qb + l32];

    // The chunks' maxima, read eight chunks at a time (a clamped chunk index
    // repeats a value, which leaves the max unchanged).
    float M[2] = {-INFINITY, -INFINITY};
    for (int c0 = 0; c0 < C; c0 += 8) {
        float mv[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                mv[u][qb] = a.part_ml[(p0 + min(c0 + u, C - 1)) * 128 + qb * 32 + l32];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) M[qb] = fmaxf(M[qb], mv[u][qb]);
    }
    float L[2] = {0.f, 0.f};
    float O[DB][2][16];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[db][qb][e] = 0.f;
    // Two chunks per iteration keep twice the partial loads in flight.
#pragma unroll 2
    for (int c = 0; c < C; ++c) {
        const float *pml = a.part_ml + (p0 + c) * 128;
        float w[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float mc = pml[qb * 32 + l32], lc = pml[64 + qb * 32 + l32];  // both loads unconditional
            w[qb] = mc == -INFINITY ? 0.f : lc * __builtin_amdgcn_exp2f((mc - M[qb]) * c2);
            L[qb] += w[qb];
        }
        const uint16_t *po = a.part_o + (p0 + c) * (64 * D);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) {
                    // Each partial is read once: non-temporal loads (1.4 % faster at H3).
                    const u32x4_t v = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t *>(po + (((db * 2 + qb) * 2 + h8) * 64 + lane) * 8));
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        O[db][qb][8 * h8 + 2 * q] += w[qb] * __uint_as_float(v[q] << 16);
                        O[db][qb][8 * h8 + 2 * q + 1] += w[qb] * __uint_as_float(v[q] & 0xffff0000u);
                    }
                }
            }
    }
    if (MODE == kMergeTrain) {
        // lse (log2 domain, +inf on padding rows) and O_fine (0 on padding rows).
        const size_t S_pad = size_t(a.n_t) * B;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = tile * B + 64 * qsub + 32 * qb + l32;
            const bool real = tok[qb] >= 0;
            const float inv = real ? 1.0f / L[qb] : 0.f;
            float *orow = a.ofine_out + (size_t(h) * S_pad + row) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4 *>(orow + 32 * db + 8 * i + 4 * half) =
                        make_float4(O[db][qb][4 * i] * inv, O[db][qb][4 * i + 1] * inv,
                                    O[db][qb][4 * i + 2] * inv, O[db][qb][4 * i + 3] * inv);
            if (half == 0) a.lse_out[size_t(h) * S_pad + row] = real ? M[qb] * c2 + __log2f(L[qb]) : INFINITY;
        }
    }
    if (MODE == kMergeStats) {
        // lse (log2 domain) and D_t = dout . O_fine per row; +inf / 0 on padding rows.
        const size_t S_pad = size_t(a.n_t) * B;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = tile * B + 64 * qsub + 32 * qb + l32;
            float part = 0.f;
            if (tok[qb] >= 0) {
                const uint16_t *go = a.dout + (size_t(tok[qb]) * a.ld + h) * D;
                const float inv = 1.0f / L[qb];
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
            part = xhalf_sum(part);  // both halves hold the full sum
            if (half == 0) {
                a.lse_out[size_t(h) * S_pad + row] = tok[qb] < 0 ? INFINITY : M[qb] * c2 + __log2f(L[qb]);
                a.dt_out[size_t(h) * S_pad + row] = tok[qb] < 0 ? 0.f : part;
            }
        }
        return;
    }
    const float *oc = a.o_coarse + (size_t(h) * a.n_t + tile) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if (tok[qb] < 0) continue;
        gated_row<DB>(a.out, a.gate, (size_t(tok[qb]) * a.ld + h) * D, oc, O, qb, 1.0f / L[qb], half);
    }
}

// INT8 K codes for the fine pass, one wave per 64-row block of the tiled K:
// scale = max|k| / 127 over the block (padding rows are zero), codes =
// round-half-even(k * (127 / max|k|)) clamped to [-127, 127], in fp32; a
// block with max|k| = 0 gets scale 0 and zero codes. Lane l of fragment
// (kb, c) holds the 16 codes of row 32kb + l%32, d = 32c + 16*(l/32) + e; they
// come from the bf16 fragment 2c + l/32 of the same rows, whose lanes l%32
// and l%32 + 32 hold d .. d+7 and d+8 .. d+15.
template <int D>
__global__ __launch_bounds__(256) void quant_k_kernel(const uint16_t *__restrict__ kt, int64_t n_blocks,
                                                     uint8_t *__restrict__ k8, float *__restrict__ k_scale)
{
    constexpr int NC8 = D / 32, NC = D / 16;
    const int lane = threadIdx.x % kWave, l32 = lane & 31, half = lane >> 5;
    const int64_t blk = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave;
    if (blk >= n_blocks) return;
    const uint16_t *src = kt + blk * (D / 8) * 512;
    u32x4_t raw[2][NC8][2];
    float amax = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NC8; ++c)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                    src + (kb * NC + 2 * c + half) * 512 + (l32 + 32 * j) * 8);
                raw[kb][c][j] = v;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[w] << 16)),
                                             fabsf(__uint_as_float(v[w] & 0xffff0000u))));
            }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    if (lane == 0) k_scale[blk] = amax > 0.f ? amax / 127.0f : 0.f;
    auto code = [&](float x) -> uint32_t {
        const float y = fminf(fmaxf(__builtin_rintf(x * inv), -127.f), 127.f);
        return uint32_t(int(y)) & 0xffu;
    };
    uint8_t *dst = k8 + blk * (64 * D);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NC8; ++c) {
            u32x4_t w;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    const uint32_t r0 = raw[kb][c][j][2 * t2], r1 = raw[kb][c][j][2 * t2 + 1];
                    w[2 * j + t2] = code(__uint_as_float(r0 << 16)) | code(__uint_as_float(r0 & 0xffff0000u)) << 8 |
                                    code(__uint_as_float(r1 << 16)) << 16 |
                                    code(__uint_as_float(r1 & 0xffff0000u)) << 24;
                }
            *reinterpret_cast<u32x4_t *>(dst + (kb * NC8 + c) * 1024 + lane * 16) = w;
        }
}

template <int D, int B, bool I8 = false>
void launch_fine(const FineArgs &a, hipStream_t st, bool train = false)
{
    const int items = a.H * a.n_t * (B / 64);
    if (I8) {
        KernelTimer t(K_QUANT_K, st);
        hipLaunchKernelGGL((quant_k_kernel<D>), dim3((items + 3) / 4), dim3(256), 0, st, a.kt, int64_t(items),
                           const_cast<uint8_t *>(a.k8), const_cast<float *>(a.k_scale));
    }
    if (a.chunks > 1) {
        {
            KernelTimer t(K_FINE_ATTN, st);
            hipLaunchKernelGGL((fine_attn_kernel<D, B, true, I8>), dim3(items * a.chunks), dim3(64), 0, st, a);
        }
        KernelTimer t(K_MERGE, st);
        if (train)
            hipLaunchKernelGGL((merge_kernel<D, B, kMergeTrain>), dim3((items + 3) / 4), dim3(256), 0, st, a, items);
        else
            hipLaunchKernelGGL((merge_kernel<D, B, kMergeOut>), dim3((items + 3) / 4), dim3(256), 0, st, a, items);
    } else {
        KernelTimer t(K_FINE_ATTN, st);
        hipLaunchKernelGGL((fine_attn_kernel<D, B, false, I8>), dim3(items), dim3(64), 0, st, a);
    }
}

// Statistics pass for the backward (key lists split into C > 1 chunks): the
// forward's split kernel, then a merge that writes lse and D_t per row.
template <int D, int B>
void launch_fine_stats(const FineArgs &a, hipStream_t st)
{
    const int items = a.H * a.n_t * (B / 64);
    {
        KernelTimer t(K_BWD_STATS, st);
        hipLaunchKernelGGL((fine_attn_kernel<D, B, true>), dim3(items * a.chunks), dim3(64), 0, st, a);
        hipLaunchKernelGGL((merge_kernel<D, B, kMergeStats>), dim3((items + 3) / 4), dim3(256), 0, st, a, items);
    }
}

}  // namespace

int fine_stats(const vsa_plan_info &info, const int32_t *row_src, const int32_t *block_len, int heads,
               int head_dim, int chunks, bool ref, int k, int k_ref, float scale, const void *q,
               const void *workspace, const int32_t *keep_idx, const void *dout, float *lse_out,
               float *dt_out, hipStream_t st)
{
    vsa_ws_layout L;
    compute_layout(info, heads, head_dim, chunks, &L);
    const char *ws = static_cast<const char *>(workspace);
    FineArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.kt = reinterpret_cast<const uint16_t *>(ws + L.k_tiled);
    a.vt = reinterpret_cast<const uint16_t *>(ws + L.v_tiled);
    a.row_src = row_src;
    a.block_len = block_len;
    a.keep = keep_idx;
    a.part_o = reinterpret_cast<uint16_t *>(const_cast<char *>(ws) + L.part_o);
    a.part_ml = reinterpret_cast<float *>(const_cast<char *>(ws) + L.part_ml);
    a.H = heads;
    a.ld = heads;
    a.P = info.n_prefix_tiles;
    a.n_v = info.n_video_tiles;
    a.n_t = info.n_tiles;
    a.k = k;
    a.chunks = chunks;
    a.ref = ref ? 1 : 0;
    a.list_len = ref ? k + k_ref : 0;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.dout = static_cast<const uint16_t *>(dout);
    a.lse_out = lse_out;
    a.dt_out = dt_out;
    if (a.chunks < 2) return VSA_ERR_UNSUPPORTED;  // small heads: the caller recomputes instead
    const int B = info.tile_rows;
    if (head_dim == 128) {
        if (B == 64) launch_fine_stats<128, 64>(a, st);
        else launch_fine_stats<128, 128>(a, st);
    } else {
        if (B == 64) launch_fine_stats<64, 64>(a, st);
        else launch_fine_stats<64, 128>(a, st);
    }
    return VSA_OK;
}

// Shared body of the fine entry points (ref: reference-sparsity lists; i8:
// INT8 scores). ld: heads per token row of q, gate and out (the pointers
// address the first head).
int fine_impl(const char *name, const vsa_plan_info *info, const int32_t *row_src_dev,
              const int32_t *block_len_dev, int heads, int ld, int head_dim, bool ref, bool i8, int k, int k_ref,
              float scale, int32_t split_req, const void *q, const void *workspace, size_t workspace_bytes,
              const int32_t *keep_idx_dev, const float *o_coarse_dev, const void *gate, void *out,
              void *stream, float *lse_out, float *ofine_out)
{
    if (int st = check_info(info)) return st;
    if (heads <= 0 || ld < heads) return fail(VSA_ERR_ARG, "%s: heads = %d (row stride %d)", name, heads, ld);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: head_dim = %d; supported: 64, 128", name, head_dim);
    if (k < 0 || k > info->n_video_tiles)
        return fail(VSA_ERR_ARG, "%s: k = %d outside [0, %d]", name, k, info->n_video_tiles);
    if (ref && (k_ref < 0 || k_ref > info->n_prefix_tiles))
        return fail(VSA_ERR_ARG, "%s: k_ref = %d outside [0, %d]", name, k_ref, info->n_prefix_tiles);
    if (!ref && info->n_prefix_tiles == 0 && k == 0 && info->n_video_tiles > 0)
        return fail(VSA_ERR_ARG, "%s: empty key set: no prefix tiles and k = 0", name);
    if (ref && k + k_ref == 0)
        return fail(VSA_ERR_ARG, "%s: empty key set: k_ref = k_gen = 0", name);
    if (!row_src_dev || !block_len_dev || !q || !workspace || !o_coarse_dev || !gate || !out)
        return fail(VSA_ERR_ARG, "%s: null device pointer", name);
    if ((ref ? k + k_ref : k) > 0 && !keep_idx_dev)
        return fail(VSA_ERR_ARG, "%s: keep_idx is null", name);
    if (!std::isfinite(scale)) return fail(VSA_ERR_ARG, "%s: scale is not finite", name);
    int chunks = 0;
    if (int st = resolve_split(*info, head_dim, split_req, &chunks)) return st;
    vsa_ws_layout L;
    compute_layout(*info, heads, head_dim, chunks, &L);
    if (workspace_bytes < L.total_bytes)
        return fail(VSA_ERR_ARG, "%s: workspace has %zu bytes, needs %zu", name, workspace_bytes,
                    L.total_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(VSA_ERR_ARG, "%s: workspace must be 256-byte aligned", name);
    // A head's tile-ordered K (or V) is addressed through one buffer resource.
    if (int64_t(info->rows_padded) * head_dim * 2 >= (int64_t(1) << 32))
        return fail(VSA_ERR_UNSUPPORTED, "%s: %lld padded rows x head_dim %d exceed 4 GiB per head", name,
                    (long long)info->rows_padded, head_dim);
    const int64_t items = int64_t(heads) * info->n_tiles * (info->tile_rows / 64);
    if (items * chunks >= (int64_t(1) << 31))
        return fail(VSA_ERR_UNSUPPORTED, "%s: too many work items (%lld)", name,
                    (long long)(items * chunks));
    if (int st = check_device()) return st;

    char *ws = static_cast<char *>(const_cast<void *>(workspace));
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
    a.part_o = reinterpret_cast<uint16_t *>(ws + L.part_o);
    a.part_ml = reinterpret_cast<float *>(ws + L.part_ml);
    a.lse_out = lse_out;
    a.ofine_out = ofine_out;
    const bool train = lse_out && ofine_out && chunks > 1;
    a.k8 = reinterpret_cast<const uint8_t *>(ws + L.k_i8);
    a.k_scale = reinterpret_cast<const float *>(ws + L.k_scale);
    a.H = heads;
    a.ld = ld;
    a.P = info->n_prefix_tiles;
    a.n_v = info->n_video_tiles;
    a.n_t = info->n_tiles;
    a.k = k;
    a.chunks = chunks;
    a.ref = ref ? 1 : 0;
    a.list_len = ref ? k + k_ref : 0;
    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(float(head_dim));
    a.scale_log2e = sc * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int B = info->tile_rows;
    if (head_dim == 128) {
        if (B == 64) i8 ? launch_fine<128, 64, true>(a, st, train) : launch_fine<128, 64>(a, st, train);
        else i8 ? launch_fine<128, 128, true>(a, st, train) : launch_fine<128, 128>(a, st, train);
    } else {
        if (B == 64) i8 ? launch_fine<64, 64, true>(a, st, train) : launch_fine<64, 64>(a, st, train);
        else i8 ? launch_fine<64, 128, true>(a, st, train) : launch_fine<64, 128>(a, st, train);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VSA_ERR_DEVICE, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
    return VSA_OK;
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_sparse_attn_fwd(const vsa_plan_info *info, const int32_t *row_src_dev,
                                   const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                   int32_t k, float scale, int32_t split_chunks, const void *q,
                                   const void *workspace, size_t workspace_bytes,
                                   const int32_t *keep_idx_dev, const float *o_coarse_dev,
                                   const void *gate, void *out, void *stream)
{
    clear_error();
    return fine_impl("vsa_sparse_attn_fwd", info, row_src_dev, block_len_dev, heads, heads, head_dim, false,
                     false, k, 0, scale, split_chunks, q, workspace, workspace_bytes, keep_idx_dev,
                     o_coarse_dev, gate, out, stream, nullptr, nullptr);
}

extern "C" int vsa_sparse_attn_fwd_ref(const vsa_plan_info *info, const int32_t *row_src_dev,
                                       const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                       int32_t k_ref, int32_t k_gen, float scale,
                                       int32_t split_chunks, const void *q,
                                       const void *workspace, size_t workspace_bytes,
                                       const int32_t *keep_idx_dev, const float *o_coarse_dev,
                                       const void *gate, void *out, void *stream)
{
    clear_error();
    return fine_impl("vsa_sparse_attn_fwd_ref", info, row_src_dev, block_len_dev, heads, heads, head_dim,
                     true, false, k_gen, k_ref, scale, split_chunks, q, workspace, workspace_bytes,
                     keep_idx_dev, o_coarse_dev, gate, out, stream, nullptr, nullptr);
}

extern "C" int vsa_sparse_attn_fwd_i8(const vsa_plan_info *info, const int32_t *row_src_dev,
                                      const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                      int32_t k_ref, int32_t k_gen, float scale,
                                      int32_t split_chunks, const void *q,
                                      void *workspace, size_t workspace_bytes,
                                      const int32_t *keep_idx_dev, const float *o_coarse_dev,
                                      const void *gate, void *out, void *stream)
{
    clear_error();
    return fine_impl("vsa_sparse_attn_fwd_i8", info, row_src_dev, block_len_dev, heads, heads, head_dim,
                     k_ref >= 0, true, k_gen, k_ref < 0 ? 0 : k_ref, scale, split_chunks, q, workspace,
                     workspace_bytes, keep_idx_dev, o_coarse_dev, gate, out, stream, nullptr, nullptr);
}
