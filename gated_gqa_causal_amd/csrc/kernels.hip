// kernels.hip -- gfx950 (CDNA4) kernels for gated GQA causal attention prefill.
//
// Three kernels run on the caller's stream:
//   kv_prologue  : (1+w) RMSNorm + partial RoPE of every key once per KV head
//                  (the QSA kernel page, "What changed": all query heads of a
//                  KV head read the same prepared key), and V transposed into
//                  MFMA-ready key tiles.  Writes the context's workspace.
//   mask_pack    : masked path only.  uint8 [S][S] visibility -> one bit per
//                  (row, key) with causality folded in, plus a per (64-row
//                  block, 32-key tile) flag used to skip fully hidden tiles.
//   attn_fwd     : one workgroup = 4 waves = 64 query rows x up to 4 query
//                  heads of one KV head.  Each wave owns 64 rows of one head:
//                  it norms and rotates its own queries, walks the key tiles
//                  0..diagonal in ascending order (online softmax, the
//                  attention-tile page's "Kernel change" recurrence), and
//                  applies the sigmoid gate in the epilogue.
//
// Rounding points follow the QSA kernel page ("Semantics"; final commit
// message): norms cast once, cos/sin cast to bf16 and the rotation done in
// bf16, the score rounded to bf16 before the exact 1/16 scale, the weights
// rounded to bf16 before the context product, the context rounded, the
// sigmoid rounded before the final product.  The GPU's online softmax rounds
// the unnormalised weight exp2(y - m) and divides by the fp32 row sum at the
// end, where the plain definition rounds normalised weights; the two agree to
// a bf16 rounding per weight.
//
// MFMA orientation: scores are computed transposed, S^T[key][query] =
// K . Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims, B = 16 dims x
// 32 queries).  The accumulator layout then gives each lane one query column
// and 16 of the tile's 32 keys, so the row max and row sum are in-lane plus
// one exchange with lane^32, and the weights feed the P.V MFMA as its B
// operand with no data movement.  The context is computed transposed too,
// O^T[d][query] = V^T . P^T, with A = V^T read from a transposed copy of V.
// The key order inside each 16-key group of that copy is
// [0..3, 8..11, 4..7, 12..15], matching the accumulator rows a lane holds.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = 256;          // head dim
constexpr int HALF_R = 32;      // rotary pairs (rotary dim 64)
constexpr int KT = 32;          // keys per tile
constexpr int QW = 64;          // query rows per attention workgroup
constexpr float LOG2E = 1.4426950408889634f;
// Scores are x = bf16(q.k); the softmax runs on y = x * (log2(e) / 16).
constexpr float SCALE_LOG2 = LOG2E * 0.0625f;
// The running max is only moved when a tile's max exceeds it by more than
// 8 in the log2 domain (weights then stay below 2^8).  The result is the same
// softmax; the rescale of the 256-wide accumulator becomes rare.
constexpr float TAU_X = 8.0f / SCALE_LOG2;

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }
__device__ __forceinline__ float rbf(float a) { return bf2f(f2bf(a)); }

__device__ __forceinline__ float word_f(const uint4 &u, int t)
{
    const uint32_t w = (t < 2) ? u.x : (t < 4) ? u.y : (t < 6) ? u.z : u.w;
    return (t & 1) ? hi_f(w) : lo_f(w);
}

// ---------------------------------------------------------------------------
// K/V prologue.  grid (Tpad/32, Hkv), 256 threads.
// Both outputs are stored as 16 KB tiles of 32 keys in the order the attention
// kernel's MFMA operand reads want them in LDS ("chunk-major": the 16-byte
// chunk index outermost), so a tile moves to LDS as one contiguous copy and
// every 16-lane group of an operand read touches 256 contiguous LDS bytes.
// Kp tile (key r, dim d): 16-byte piece (d / 8) * 32 + r, element d % 8.
// Vt tile (dim d, key slot s): piece (s / 8) * 256 + d, element s % 8, where
// slot s holds key [0..3, 8..11, 4..7, 12..15] of each 16 (V transposed, keys
// permuted to match the score accumulator layout).  Keys past T are zero.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int vt_key_of_pos(int pos)
{
    const int w = pos & 15;
    const int k16 = (w < 4) ? w : (w < 8) ? w + 4 : (w < 12) ? w - 4 : w;
    return (pos & ~15) | k16;
}

__global__ __launch_bounds__(256) void kv_prologue(KvPrologueParams p)
{
    __shared__ __align__(16) uint16_t ks[KT][D + 8];
    __shared__ __align__(16) uint16_t vs[KT][D + 8];
    __shared__ float rs[KT];
    const int tile = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    const int t0 = tile * KT;

    for (int it = 0; it < 4; ++it) {
        const int idx = it * 256 + tid, r = idx >> 5, ch = idx & 31, key = t0 + r;
        uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (key < p.T) {
            const size_t off = ((size_t)key * p.Hkv + c) * D + ch * 8;
            kv = *reinterpret_cast<const uint4 *>(p.k + off);
            vv = *reinterpret_cast<const uint4 *>(p.v + off);
        }
        *reinterpret_cast<uint4 *>(&ks[r][ch * 8]) = kv;
        *reinterpret_cast<uint4 *>(&vs[r][ch * 8]) = vv;
    }
    __syncthreads();

    // Sum of squares in ascending dimension order, one thread per key.
    if (tid < KT) {
        float ss = 0.0f;
        for (int d = 0; d < D; ++d) {
            const float x = bf2f(ks[tid][d]);
            ss += x * x;
        }
        rs[tid] = 1.0f / sqrtf(ss / (float)D + p.eps);
    }
    __syncthreads();

    {
        // Thread owns dims sub + 8*s of key row r; pairs (j, j+32) are s, s+4.
        const int r = tid >> 3, sub = tid & 7, key = t0 + r;
        const float rr = rs[r];
        float n[32];
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int d = sub + 8 * s;
            n[s] = rbf((bf2f(ks[r][d]) * rr) * (1.0f + bf2f(p.wk[d])));
        }
        if (key < p.T) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int j = sub + 8 * s;
                const float cj = rbf(p.cos_tab[(size_t)key * HALF_R + j]);
                const float sj = rbf(p.sin_tab[(size_t)key * HALF_R + j]);
                const float a = n[s], b = n[s + 4];
                n[s] = rbf(rbf(a * cj) + rbf(-b * sj));
                n[s + 4] = rbf(rbf(b * cj) + rbf(a * sj));
            }
        }
#pragma unroll
        for (int s = 0; s < 32; ++s)
            ks[r][sub + 8 * s] = (key < p.T) ? f2bf(n[s]) : (uint16_t)0;
    }
    __syncthreads();

    const size_t tile_off = ((size_t)c * (p.Tpad / KT) + tile) * (size_t)(KT * D);
    uint4 *kdst = reinterpret_cast<uint4 *>(p.kp + tile_off);
    for (int it = 0; it < 4; ++it) {
        const int piece = it * 256 + tid, ch = piece >> 5, r = piece & 31;
        kdst[piece] = *reinterpret_cast<const uint4 *>(&ks[r][ch * 8]);
    }

    uint4 *vdst = reinterpret_cast<uint4 *>(p.vt + tile_off);
    for (int q = 0; q < 4; ++q) {
        const int d = tid;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = vs[vt_key_of_pos(8 * q + 2 * e)][d];
            const uint32_t b = vs[vt_key_of_pos(8 * q + 2 * e + 1)][d];
            w[e] = a | (b << 16);
        }
        vdst[q * 256 + d] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Debug: prepared keys from the tiled layout back to plain [Hkv][T][D].
// grid (ceil(T/32), Hkv), 256 threads.
__global__ __launch_bounds__(256) void kp_unpack(const uint16_t *kp, int Tpad, int T, uint16_t *out)
{
    const int tile = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    const uint4 *src = reinterpret_cast<const uint4 *>(kp + ((size_t)c * (Tpad / KT) + tile) * (size_t)(KT * D));
    for (int it = 0; it < 4; ++it) {
        const int piece = it * 256 + tid, ch = piece >> 5, r = piece & 31, key = tile * KT + r;
        if (key < T)
            *reinterpret_cast<uint4 *>(out + ((size_t)c * T + key) * D + ch * 8) = src[piece];
    }
}

// ---------------------------------------------------------------------------
// Mask packing.  grid (ceil(W/256), nrb), 256 threads; thread = (row block, word).
// bits[row][w] bit b = mask[row][32w+b] != 0 && 32w+b <= row && 32w+b < S.
// tilevis[rb][w] = any bit of the 64 x 32 block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nz_bits4(uint32_t u)
{
    return ((u & 0x000000ffu) ? 1u : 0u) | ((u & 0x0000ff00u) ? 2u : 0u) |
           ((u & 0x00ff0000u) ? 4u : 0u) | ((u & 0xff000000u) ? 8u : 0u);
}

__global__ __launch_bounds__(256) void mask_pack(MaskPackParams p)
{
    const int w = blockIdx.x * 256 + threadIdx.x;
    const int rb = blockIdx.y;
    if (w >= p.W)
        return;
    const int key0 = 32 * w;
    uint32_t any = 0;
    for (int r = 0; r < QW; ++r) {
        const int row = rb * QW + r;
        if (row >= p.S)
            break;
        uint32_t word = 0;
        if (key0 <= row) {
            const uint8_t *src = p.mask + (size_t)row * p.S + key0;
            if (p.vec16 && key0 + 32 <= p.S) {
                const uint4 a = *reinterpret_cast<const uint4 *>(src);
                const uint4 b = *reinterpret_cast<const uint4 *>(src + 16);
                word = nz_bits4(a.x) | (nz_bits4(a.y) << 4) | (nz_bits4(a.z) << 8) |
                       (nz_bits4(a.w) << 12) | (nz_bits4(b.x) << 16) | (nz_bits4(b.y) << 20) |
                       (nz_bits4(b.z) << 24) | (nz_bits4(b.w) << 28);
            } else {
                for (int b = 0; b < 32; ++b)
                    if (key0 + b < p.S && src[b] != 0)
                        word |= 1u << b;
            }
            const int last = row - key0;               // keys key0..row are causal
            if (last < 31)
                word &= (2u << last) - 1u;
        }
        p.bits[(size_t)row * p.W + w] = word;
        any |= word;
    }
    p.tilevis[(size_t)rb * p.W + w] = any ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Query prologue of one wave: loads the q half of 32 rows of head h, applies
// (1+w) RMSNorm (sum of squares in ascending dimension order, the same chain
// as the key prologue) and partial RoPE, and leaves the MFMA B-operand
// fragments in qf[c]: lane (j = lane & 31, hh = lane >> 5) holds dims
// 16c + 8hh .. +7 of query row r0 + j.  Rows at or past S are zero.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_queries(const AttnParams &p, int r0, int h, int lane,
                                             uint4 (&qf)[16])
{
    const int j = lane & 31, hh = lane >> 5;
    const int row = r0 + j;
    const bool ok = row < p.S;
    const uint16_t *src = p.qg + (((size_t)(ok ? row : 0) * p.Hq + h) * 2) * D;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        qf[c] = *reinterpret_cast<const uint4 *>(src + 16 * c + 8 * hh);
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const uint4 own = qf[c];
        uint4 oth;
        oth.x = __shfl_xor(own.x, 32);
        oth.y = __shfl_xor(own.y, 32);
        oth.z = __shfl_xor(own.z, 32);
        oth.w = __shfl_xor(own.w, 32);
        const uint4 first = hh ? oth : own;
        const uint4 second = hh ? own : oth;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float x = word_f(first, t);
            ss += x * x;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float x = word_f(second, t);
            ss += x * x;
        }
    }
    const float rr = 1.0f / sqrtf(ss / (float)D + p.eps);
    // Dims 0..63 (chunks 0..3) hold the rotary pairs (d, d+32) = chunks
    // (c, c+2); the remaining chunks are only normalised.
    {
        float n[4][8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 wv = *reinterpret_cast<const uint4 *>(p.wq + 16 * c + 8 * hh);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                n[c][t] = rbf((word_f(qf[c], t) * rr) * (1.0f + word_f(wv, t)));
        }
        const int pos = p.q_base + (ok ? row : 0);
        const float *ct = p.cos_tab + (size_t)pos * HALF_R;
        const float *st = p.sin_tab + (size_t)pos * HALF_R;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float4 c0 = *reinterpret_cast<const float4 *>(ct + 16 * c + 8 * hh);
            const float4 c1 = *reinterpret_cast<const float4 *>(ct + 16 * c + 8 * hh + 4);
            const float4 s0 = *reinterpret_cast<const float4 *>(st + 16 * c + 8 * hh);
            const float4 s1 = *reinterpret_cast<const float4 *>(st + 16 * c + 8 * hh + 4);
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float cj = rbf(cv[t]), sj = rbf(sv[t]);
                const float a = n[c][t], bb = n[c + 2][t];
                n[c][t] = rbf(rbf(a * cj) + rbf(-bb * sj));
                n[c + 2][t] = rbf(rbf(bb * cj) + rbf(a * sj));
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            qf[c] = make_uint4(pack2(n[c][0], n[c][1]), pack2(n[c][2], n[c][3]),
                               pack2(n[c][4], n[c][5]), pack2(n[c][6], n[c][7]));
    }
#pragma unroll
    for (int c = 4; c < 16; ++c) {
        const uint4 wv = *reinterpret_cast<const uint4 *>(p.wq + 16 * c + 8 * hh);
        float n[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            n[t] = rbf((word_f(qf[c], t) * rr) * (1.0f + word_f(wv, t)));
        qf[c] = make_uint4(pack2(n[0], n[1]), pack2(n[2], n[3]), pack2(n[4], n[5]), pack2(n[6], n[7]));
    }
    if (!ok) {
#pragma unroll
        for (int c = 0; c < 16; ++c)
            qf[c] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Debug: prepared queries in a plain [rows][Hq][D] layout.
// grid (ceil(S/32), ceil(Hq/4)), 256 threads: wave = one head, 32 rows.
__global__ __launch_bounds__(256) void q_prologue_debug(AttnParams p, uint16_t *qp)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y * 4 + wave;
    if (h >= p.Hq)
        return;
    const int r0 = blockIdx.x * 32;
    uint4 qf[16];
    load_queries(p, r0, h, lane, qf);
    const int j = lane & 31, hh = lane >> 5;
    const int row = r0 + j;
    if (row >= p.S)
        return;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        *reinterpret_cast<uint4 *>(qp + ((size_t)row * p.Hq + h) * D + 16 * c + 8 * hh) = qf[c];
}

// ---------------------------------------------------------------------------
// Attention.  Workgroup = 8 waves = 64 query rows x 4 query heads of one KV
// head; wave w owns head (w & 3) and rows r0 + 32 * (w >> 2) .. +31.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

constexpr int AW = 8;                  // waves per attention workgroup
constexpr int ATHREADS = 64 * AW;
constexpr int QR = 32;                 // query rows per wave
constexpr int MAX_TILES = 32768 / KT;  // tile list capacity (token cap / 32)

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane L
// writes LDS bytes [lds + 16 L, lds + 16 L + 16) from gbase + voff.  gbase and
// lds must be wave-uniform.  Issued through inline asm so the compiler does
// not guard later LDS reads of *other* buffers with a wait on this load; the
// caller orders it with an explicit s_waitcnt vmcnt before the barrier that
// publishes the buffer.
// M0 is reserved by the compiler: it is saved and restored around the copy.
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(voff), "s"(gbase)
                 : "memory");
}
// Same for 4 bytes per lane (global_load_lds_dword): lane L writes lds + 4 L.
__device__ __forceinline__ void dma4(const void *gbase, uint32_t voff, uint32_t lds)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(voff), "s"(gbase)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}

// Sum and max of a value with its partner lane (lane ^ 32).  v_permlane32_swap
// exchanges the upper half of one register with the lower half of the other;
// fed the same value twice, each lane ends with its own value in one result
// and the partner's in the other, whichever way round.
__device__ __forceinline__ float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Per-lane LDS byte offsets of the MFMA operand fragments.
// K fragment (dims 16c + 8hh .. +7 of key row j): piece (2c + hh) * 32 + j
//   -> hh * 512 + j * 16 + 1024 * c.
// V^T fragment (dim row 32db + j, key slots 16kc + 8hh .. +7):
//   piece (2kc + hh) * 256 + 32db + j -> hh * 4096 + j * 16 + 8192 * kc + 512 * db.
struct FragOffsets {
    int k;
    int v;
};

__device__ __forceinline__ FragOffsets frag_offsets(int j, int hh)
{
    return FragOffsets{hh * 512 + j * 16, hh * 4096 + j * 16};
}

// S^T = K . Q^T for one tile: lane holds query j, keys 8g + 4hh + r (e = 4g + r).
__device__ __forceinline__ void tile_scores(const char *kb, const FragOffsets &fo, const uint4 (&qf)[16],
                                            f32x16 &s)
{
#pragma unroll
    for (int e = 0; e < 16; ++e)
        s[e] = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        // At most four fragments in flight (the Q fragments and the context
        // accumulators hold 192 of the 256 registers).
        if ((c & 3) == 0)
            __builtin_amdgcn_sched_barrier(0);
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb + fo.k + 1024 * c);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, __builtin_bit_cast(bf16x8, qf[c]), s, 0, 0, 0);
    }
}

// Scores of hidden keys become -inf (they round to bf16 -inf and weigh exactly
// 0).  vis bit kk = key kk of the tile is visible to this lane's query; this
// lane holds keys 8g + 4hh + r.
__device__ __forceinline__ void hide_scores(f32x16 &s, uint32_t vis, int hh)
{
    const uint32_t vh = vis >> (4 * hh);
#pragma unroll
    for (int e = 0; e < 16; ++e)
        s[e] = ((vh >> (8 * (e >> 2) + (e & 3))) & 1u) ? s[e] : -INFINITY;
}

// Online softmax of one tile's scores -> bf16 weights pk (relative to the
// running max), updating (m, l) and rescaling O when the max moves.
__device__ __forceinline__ void tile_softmax(const f32x16 &s, float &m, float &l, uint32_t (&pk)[8],
                                             f32x16 (&o)[8])
{
    float x[16];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t w = pack2(s[2 * q], s[2 * q + 1]);     // bf16(q . k)
        x[2 * q] = lo_f(w);
        x[2 * q + 1] = hi_f(w);
    }
    float mt = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2)
        mt = fmaxf(fmaxf(mt, x[e]), x[e + 1]);
    mt = fmaxf(mt, x[15]);
    mt = pair_max(mt);
    const float mo = m;
    const float mn = (mt > mo + TAU_X) ? mt : mo;
    const float alpha = (mn == mo) ? 1.0f : __builtin_amdgcn_exp2f((mo - mn) * SCALE_LOG2);
    m = mn;
    const float base = (mn == -INFINITY) ? 0.0f : mn * SCALE_LOG2;
    float ls = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * q], SCALE_LOG2, -base));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * q + 1], SCALE_LOG2, -base));
        ls += p0;
        ls += p1;
        pk[q] = pack2(p0, p1);
    }
    l = l * alpha + ls;
    if (__builtin_expect(__any(alpha != 1.0f), 0)) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                o[db][e] *= alpha;
    }
}

// O^T += V^T . P^T; P chunk kc = keys 16kc .. 16kc+15 = pk[4kc .. 4kc+3].
__device__ __forceinline__ void tile_context(const char *vb, const FragOffsets &fo, const uint32_t (&pk)[8],
                                             f32x16 (&o)[8])
{
    const uint4 p0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    const uint4 p1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        if ((db & 1) == 0)
            __builtin_amdgcn_sched_barrier(0);
        const bf16x8 v0 = *reinterpret_cast<const bf16x8 *>(vb + fo.v + 512 * db);
        const bf16x8 v1 = *reinterpret_cast<const bf16x8 *>(vb + fo.v + 8192 + 512 * db);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, __builtin_bit_cast(bf16x8, p0), o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, __builtin_bit_cast(bf16x8, p1), o[db], 0, 0, 0);
    }
}

// The matrix half of an interval: O += V^T . P^T for the previous tile and
// S^T = K . Q^T for the current one, issued alternately.  The 16 score MFMAs
// form one accumulation chain; putting an independent context MFMA between
// consecutive links keeps the matrix pipe busy while each link completes.
__device__ __forceinline__ void matrix_half(const char *kb, const char *vb, const FragOffsets &fo,
                                            const uint4 (&qf)[16], const uint32_t (&pk)[8], f32x16 (&o)[8],
                                            f32x16 &s)
{
    const uint4 p0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    const uint4 p1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int e = 0; e < 16; ++e)
        s[e] = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        // Two (score, context) pairs of fragments in flight at a time.
        if ((c & 1) == 0)
            __builtin_amdgcn_sched_barrier(0);
        const int db = c >> 1, kc = c & 1;
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb + fo.k + 1024 * c);
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vb + fo.v + 8192 * kc + 512 * db);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, __builtin_bit_cast(bf16x8, qf[c]), s, 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, kc ? p1 : p0), o[db], 0,
                                                       0, 0);
    }
}

// Key walk.  Interval k (between two workgroup barriers) reads K(k) and
// V(k-1) from LDS while K(k+2) and V(k+1) load into the third buffers (three
// per operand: loads run two intervals ahead of their use).  Each
// wave's tile work has a matrix half M(k) = [O += V(k-1) P(k-1); S = K(k) Q^T]
// and a vector half V(k) = softmax(S) -> P(k).  Group A (waves 0..3) runs
// M(k) then V(k) in interval k; group B (waves 4..7) runs V(k-1) then M(k).
// Waves w and w + 4 share a SIMD, so in each half of an interval one of them
// feeds the matrix pipe while the other runs the softmax.
template <bool MASKED>
__global__ __attribute__((amdgpu_flat_work_group_size(ATHREADS, ATHREADS), amdgpu_waves_per_eu(2, 2)))
void attn_fwd(AttnParams p)
{
    __shared__ __align__(16) uint16_t kbuf[3][KT * D];
    __shared__ __align__(16) uint16_t vbuf[3][D * KT];
    __shared__ uint32_t bitsbuf[4][QW];
    __shared__ int tile_list[MASKED ? MAX_TILES : 1];
    __shared__ int tile_count;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;                       // 0: rows r0.. (group A), 1: rows r0+32.. (B)
    const int j = lane & 31, hh = lane >> 5;

    // Heaviest row blocks first (longest key walks), then KV head, then head group.
    const int per_rb = p.Hkv * p.n_hg;
    const int rb = p.nrb - 1 - (int)(blockIdx.x / per_rb);
    const int rem = blockIdx.x % per_rb;
    const int kvh = rem / p.n_hg, hg = rem % p.n_hg;
    const int gidx = hg * 4 + (wave & 3);
    const int r0 = rb * QW + QR * grp;               // this wave's first window row
    const bool active = gidx < p.G && r0 < p.S;
    const int h = kvh * p.G + (active ? gidx : 0);

    const int P0 = p.q_base + rb * QW;               // workgroup's first absolute position
    const int ntiles = min(P0 + QW - 1, p.T - 1) / KT + 1;
    const int diag = (P0 + QR * grp) / KT;           // the wave's diagonal tile (its last)

    // The workgroup's tile sequence: every tile up to the diagonal, or (masked)
    // the tiles with a visible key for some row of the block, ascending.
    int n = ntiles;
    if (MASKED) {
        if (wave == 0) {
            int cnt = 0;
            for (int t0 = 0; t0 < ntiles; t0 += 64) {
                const int t = t0 + lane;
                const bool on = t < ntiles && p.tilevis[(size_t)rb * p.W + t] != 0;
                const uint64_t bal = __ballot(on);
                const int at = cnt + __popcll(bal & ((1ull << lane) - 1ull));
                if (on)
                    tile_list[at] = t;
                cnt += __popcll(bal);
            }
            if (lane == 0)
                tile_count = cnt;
        }
        __syncthreads();
        n = tile_count;
    }
    auto tile_at = [&](int u) -> int { return MASKED ? tile_list[u] : u; };

    // Each of the 8 waves moves 2 KB of each 16 KB tile straight from global
    // memory into LDS (global_load_lds_dwordx4: lane L of an instruction
    // writes the 16 bytes at LDS base + 16 L, from consecutive addresses).
    auto load_tile = [&](const uint16_t *base, int tile, uint16_t *dst) {
        tile = __builtin_amdgcn_readfirstlane(tile);
        const uint16_t *src = base + ((size_t)kvh * (p.Tpad / KT) + tile) * (size_t)(KT * D);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int nn = wave * 2 + i;
            dma16(src, (uint32_t)(nn * 1024 + lane * 16), lds_addr(dst) + nn * 1024);
        }
    };
    // Masked path: the 64 rows' visibility words of a tile, next to its K
    // load; wave w moves the words of rows 8w .. 8w+7 (lanes outside that
    // range are masked off, lane L still writes word L).
    auto load_bits = [&](int tile, uint32_t *dst) {
        if (MASKED) {
            tile = __builtin_amdgcn_readfirstlane(tile);
            if ((lane >> 3) == wave) {
                const int row = min(rb * QW + lane, p.S - 1);   // rows past S read a real row
                dma4(p.bits, (uint32_t)(((size_t)row * p.W + tile) * 4), lds_addr(dst));
            }
        }
    };
    // Every interval issues the same loads per wave (tiles past the end are
    // clamped to the last one and land in a buffer nobody reads), so the
    // wait for the previous interval's loads is one fixed count.
    auto tile_clamped = [&](int u) { return tile_at(min(u, n - 1)); };

    if (n > 0) {
        load_tile(p.kp, tile_clamped(0), kbuf[0]);
        load_bits(tile_clamped(0), bitsbuf[0]);
        load_tile(p.kp, tile_clamped(1), kbuf[1]);
        load_bits(tile_clamped(1), bitsbuf[1]);
        load_tile(p.vt, tile_clamped(0), vbuf[0]);
    }

    // Every wave prepares its fragments (an idle wave's are never used); keeping
    // the definition unconditional keeps them in registers.
    uint4 qf[16];
    load_queries(p, r0, h, lane, qf);
    const FragOffsets fo = frag_offsets(j, hh);
    // Causal visibility inside the wave's diagonal tile (keys and rows both
    // start at 32 * diag): bit kk set iff kk <= j.
    const uint32_t diag_vis = (j == 31) ? 0xffffffffu : ((2u << j) - 1u);

    f32x16 o[8];
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            o[db][e] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        s[e] = 0.0f;
    uint32_t pk[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Matrix half M(k) and vector half V(u) of this wave.  Tiles past the
    // wave's diagonal get all-hidden scores, an exact no-op (running max
    // unchanged, alpha = 1, P = 0), so both halves run on every tile of the
    // workgroup's walk; an idle wave's results are never stored.
    auto scores = [&](int k) { tile_scores(reinterpret_cast<const char *>(kbuf[k % 3]), fo, qf, s); };
    auto context = [&](int k) { tile_context(reinterpret_cast<const char *>(vbuf[k % 3]), fo, pk, o); };
    auto vector_half = [&](int u) {
        const int t = tile_at(u);
        if (MASKED || t >= diag) {
            uint32_t vis = (t == diag) ? diag_vis : (t < diag ? 0xffffffffu : 0u);
            if (MASKED)
                vis &= bitsbuf[u & 3][QR * grp + j];
            hide_scores(s, vis, hh);
        }
        tile_softmax(s, m, l, pk, o);
    };
    // Interval k's loads: K(k+2) (+ its row words) and V(k+1).
    auto loads = [&](int k) {
        load_tile(p.kp, tile_clamped(k + 2), kbuf[(k + 2) % 3]);
        load_bits(tile_clamped(k + 2), bitsbuf[(k + 2) & 3]);
        load_tile(p.vt, tile_clamped(k + 1), vbuf[(k + 1) % 3]);
    };
    // Wait for the previous interval's loads (this interval's stay in flight:
    // 4 per wave, 5 with the mask words), then the barrier.
    auto close_interval = [&]() {
        if (MASKED)
            asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        __syncthreads();
    };

    if (n > 0) {
        if (grp == 0) {
            // Group A: interval k = [O += V(k-1) P(k-1); S(k)] then softmax(k).
            loads(0);
            scores(0);
            vector_half(0);
            close_interval();
#pragma clang loop unroll(disable)
            for (int k = 1; k < n; ++k) {
                loads(k);
                matrix_half(reinterpret_cast<const char *>(kbuf[k % 3]),
                            reinterpret_cast<const char *>(vbuf[(k - 1) % 3]), fo, qf, pk, o, s);
                vector_half(k);
                close_interval();
            }
            loads(n);
            context(n - 1);
            close_interval();
        } else {
            // Group B: interval k = softmax(k-1) then [O += V(k-1) P(k-1); S(k)].
            loads(0);
            scores(0);
            close_interval();
#pragma clang loop unroll(disable)
            for (int k = 1; k < n; ++k) {
                loads(k);
                vector_half(k - 1);
                matrix_half(reinterpret_cast<const char *>(kbuf[k % 3]),
                            reinterpret_cast<const char *>(vbuf[(k - 1) % 3]), fo, qf, pk, o, s);
                close_interval();
            }
            loads(n);
            vector_half(n - 1);
            context(n - 1);
            close_interval();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    if (!active)
        return;

    // Epilogue: ctx = bf16(O / l), out = bf16(ctx * bf16(sigmoid(gate))).
    const float lt = pair_sum(l);
    const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
    const int row = r0 + j;
    if (row >= p.S)
        return;
    const uint16_t *gsrc = p.qg + (((size_t)row * p.Hq + h) * 2 + 1) * D;
    uint16_t *dst = p.out + ((size_t)row * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * hh;
            const uint2 gw = *reinterpret_cast<const uint2 *>(gsrc + d0);
            const float gv[4] = {lo_f(gw.x), hi_f(gw.x), lo_f(gw.y), hi_f(gw.y)};
            float ov[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ctx = rbf(o[db][4 * g + r] * inv);
                // Hardware reciprocal (exact at 1 and 2: a saturated logit gives
                // exactly 1, a zero logit exactly 1/2).
                const float sg = rbf(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[r] * LOG2E)));
                ov[r] = ctx * sg;
            }
            *reinterpret_cast<uint2 *>(dst + d0) = make_uint2(pack2(ov[0], ov[1]), pack2(ov[2], ov[3]));
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_kv_prologue(const KvPrologueParams &p, int ntiles, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_prologue, dim3(ntiles, p.Hkv), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mask_pack(const MaskPackParams &p, int nrb, hipStream_t stream)
{
    hipLaunchKernelGGL(mask_pack, dim3((p.W + 255) / 256, nrb), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnParams &p, bool masked, hipStream_t stream)
{
    const int nblocks = p.nrb * p.Hkv * p.n_hg;
    if (masked)
        hipLaunchKernelGGL(attn_fwd<true>, dim3(nblocks), dim3(ATHREADS), 0, stream, p);
    else
        hipLaunchKernelGGL(attn_fwd<false>, dim3(nblocks), dim3(ATHREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_kp_unpack(const uint16_t *kp, int Tpad, int T, int Hkv, uint16_t *out, hipStream_t stream)
{
    hipLaunchKernelGGL(kp_unpack, dim3((T + KT - 1) / KT, Hkv), dim3(256), 0, stream, kp, Tpad, T, out);
    return hipGetLastError();
}

hipError_t launch_q_prologue_debug(const AttnParams &p, uint16_t *qp, hipStream_t stream)
{
    hipLaunchKernelGGL(q_prologue_debug, dim3((p.S + 31) / 32, (p.Hq + 3) / 4), dim3(256), 0,
                       stream, p, qp);
    return hipGetLastError();
}

}  // namespace ga
