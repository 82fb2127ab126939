// kernels.hip -- gfx950 (CDNA4) kernels for gated GQA causal attention prefill.
//
// The kernels of a call run on the caller's stream:
//   kv_prologue  : (1+w) RMSNorm + partial RoPE of every key once per KV head
//                  (the QSA kernel page, "What changed": a key is prepared a
//                  single time and then shared by every query head of its KV
//                  group), and V transposed into MFMA-ready key tiles.  Writes
//                  the context's workspace.
//   mask_pack    : masked path only.  uint8 [S][S] visibility -> one bit per
//                  (row, key) with causality folded in, plus a per (64-row
//                  block, 32-key tile) flag used to skip fully hidden tiles.
//   kv_widen     : fp8 cache only.  e4m3 key / value rows -> the bf16 tiles.
//   attn_fwd8    : one workgroup = 8 waves = 64 query rows x up to 4 query
//                  heads of one KV head.  Each wave owns 32 rows of one head:
//                  it norms and rotates its own queries, walks the key tiles
//                  0..diagonal in ascending order (online softmax, the
//                  attention-tile page's "Kernel change" recurrence), and
//                  applies the sigmoid gate in the epilogue.
//
// Rounding points follow the QSA kernel page ("Semantics"; final commit
// message): each normalised vector rounded to bf16 a single time, cos/sin
// rounded to bf16 and the rotation done in bf16 arithmetic, the score
// rounded to bf16 before the exact 1/16 scale, the weights
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
#include <algorithm>
#include <mutex>
#include <stdint.h>

#include "kernels.h"
#include "schedule.h"

namespace ga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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
// x rounded to bf16 (nearest even), as an fp32 value: the packed convert with
// a zero low half leaves bf16(x) in the high half, which is that value.
__device__ __forceinline__ float round_op(float x)
{
    float r;
    asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(r) : "v"(x));
    return r;
}

__device__ __forceinline__ float word_f(const uint4 &u, int t)
{
    const uint32_t w = (t < 2) ? u.x : (t < 4) ? u.y : (t < 6) ? u.z : u.w;
    return (t & 1) ? hi_f(w) : lo_f(w);
}

// ---------------------------------------------------------------------------
// K/V prologue.  grid (tiles, Hkv), 256 threads: tiles tile0 .. tile0 + tiles - 1
// (keys up to T); k and v rows start at position k_row0 (0, or the first new
// key when appending to a cache).
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

// Stores 32 prepared keys (ks, bf16 rows) as one chunk-major Kp tile at kdst
// (256 threads).
__device__ __forceinline__ void write_k_tile(const uint16_t (&ks)[KT][D + 8], uint16_t *kdst, int tid)
{
    uint4 *dst = reinterpret_cast<uint4 *>(kdst);
    for (int it = 0; it < 4; ++it) {
        const int piece = it * 256 + tid, ch = piece >> 5, r = piece & 31;
        dst[piece] = *reinterpret_cast<const uint4 *>(&ks[r][ch * 8]);
    }
}

// Stores 32 values (vs, bf16 rows) as one chunk-major Vt tile at vdst: its
// 1024 16-byte pieces (q, d) = (piece / 256, piece % 256), taken by threads t
// of nthreads in steps of nthreads.
__device__ __forceinline__ void write_vt_tile(const uint16_t (&vs)[KT][D + 8], uint16_t *vdst, int t, int nthreads)
{
    uint4 *dst = reinterpret_cast<uint4 *>(vdst);
    for (int piece = t; piece < 4 * D; piece += nthreads) {
        const int q = piece >> 8, d = piece & (D - 1);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = vs[vt_key_of_pos(8 * q + 2 * e)][d];
            const uint32_t b = vs[vt_key_of_pos(8 * q + 2 * e + 1)][d];
            w[e] = a | (b << 16);
        }
        dst[piece] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Stores one tile: 32 prepared keys (ks) and 32 values (vs), bf16 rows, into
// the chunk-major Kp and Vt layouts at element offset tile_off (256 threads).
__device__ __forceinline__ void write_kv_tile(const uint16_t (&ks)[KT][D + 8], const uint16_t (&vs)[KT][D + 8],
                                              uint16_t *kp, uint16_t *vt, size_t tile_off, int tid)
{
    write_k_tile(ks, kp + tile_off, tid);
    write_vt_tile(vs, vt + tile_off, tid, 256);
}

// ---------------------------------------------------------------------------
// fp8 cache rows (the long-prompt prefill page, Kernels list: e4m3 cache rows
// with an fp32 scale each, widened to bf16).  E4M3 as the OCP 8-bit floating
// point format defines it: sign, 4 exponent bits (bias 7), 3 mantissa bits,
// subnormals at exponent 0, no infinities, S.1111.111 NaN, 448 the largest
// finite magnitude.  A row's scale is amax / 448 (1 for a zero row); a value
// is encoded from x / scale to the nearest code, ties to the even mantissa,
// magnitudes past 448 saturated; it is widened as bf16(value(code) * scale).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t enc_e4m3(float x)
{
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a == a))
        return 0x7Fu;                                    // NaN
    if (a >= 448.0f)
        return sign | 0x7Eu;                             // saturate
    if (a < 0.015625f) {                                 // below 2^-6: multiples of 2^-9
        const uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);   // exact scaling, ties to even
        return sign | m;                                 // m == 8 is the smallest normal, 0x08
    }
    const uint32_t ua = __float_as_uint(a);
    uint32_t e = (ua >> 23) - 127u + 7u;                 // 1 .. 15
    uint32_t keep = (ua >> 20) & 7u;
    const uint32_t rest = ua & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u)))
        ++keep;
    if (keep == 8u) {
        keep = 0u;
        ++e;
    }
    return sign | (e << 3) | keep;                       // a < 448 never reaches the NaN code
}

// x / sc rounded to nearest even, given y = 1 / sc rounded to nearest (one
// exact division per row instead of one per value): q = x y is within an ulp
// of the quotient, the FMA yields the remainder x - q sc exactly, and q + r y
// rounded once is the correctly rounded quotient (Markstein's theorem on
// FMA-based division; it needs the remainder to stay in the normal range,
// which holds for every quotient of 2^-11 or more when sc >= 2^-49).  The
// sign comes from x, so that x = -0 gives -0.
__device__ __forceinline__ float div_rn(float x, float sc, float y)
{
    const float q = __fmul_rn(x, y);
    const float r = __builtin_fmaf(-q, sc, x);
    return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

// Four values to e4m3 codes (byte i = value i) by the hardware's OCP e4m3
// convert, round to nearest even.
__device__ __forceinline__ uint32_t enc4_e4m3(float a, float b, float c, float d)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)lo, true);
}

__device__ __forceinline__ float dec_e4m3(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = (e == 0u) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    if ((c & 0x7Fu) == 0x7Fu)
        mag = __builtin_nanf("");
    return (c & 0x80u) ? -mag : mag;
}

// One 16-value chunk of an fp8 cache row (one key or value of one KV head)
// to e4m3 codes at dst, by 16 consecutive lanes (lane ch of the row's group
// takes chunk ch): the lanes combine their largest magnitudes with xor
// shuffles into the row's, whose scale (amax / 448; 1 for an all-zero row and
// for a row holding a NaN, where amax is NaN) the chunk's codes use; lane 0
// of the group stores the scale.  The largest magnitude is the integer max of
// the bf16 bit patterns with the sign cleared: finite magnitudes in order, inf
// above them, NaN above inf.  keep: the row is a key position to store.
__device__ __forceinline__ void fp8_row_chunk(const uint16_t *src, int ch, bool keep, uint8_t *dst, float *scale)
{
    const uint4 u0 = *reinterpret_cast<const uint4 *>(src), u1 = *reinterpret_cast<const uint4 *>(src + 8);
    const uint32_t wd[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int t = 0; t < 8; ++t)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, wd[t] & 0x7fff7fffu));
    uint32_t mx = max((uint32_t)m2.x, (uint32_t)m2.y);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    const float a = __uint_as_float(mx << 16);
    const float sc = (a > 0.0f) ? a / 448.0f : 1.0f;
    if (!keep)
        return;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (mx >= 0x2b80u && mx < 0x7f80u) {
        // Finite row with amax >= 2^-40 (sc >= 2^-49): one division for the
        // row, three operations per value.
        const float y = 1.0f / sc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w0 = wd[2 * q], w1 = wd[2 * q + 1];
            w[q] = enc4_e4m3(div_rn(lo_f(w0), sc, y), div_rn(hi_f(w0), sc, y), div_rn(lo_f(w1), sc, y),
                             div_rn(hi_f(w1), sc, y));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t we = wd[e >> 1];
            w[e >> 2] |= enc_e4m3(((e & 1) ? hi_f(we) : lo_f(we)) / sc) << (8 * (e & 3));
        }
    }
    *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    if (ch == 0)
        *scale = sc;
}

template <bool FP8>
__global__ __launch_bounds__(256) void kv_prologue(KvPrologueParams p)
{
    __shared__ __align__(16) uint16_t ks[KT][D + 8];
    __shared__ __align__(16) uint16_t vs[KT][D + 8];
    __shared__ float rs[KT];
    __shared__ float wk1[D];                     // 1 + w_k in fp32
    // tile: prepared tile written; t0: position of its first key; T: keys of
    // the sequence; raw row of position key = key + row_base.
    const int tile = p.tile0 + (int)blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    int t0 = tile * KT, T = p.T, row_base = -p.k_row0;
    if (p.tile_seg) {
        // sequence sq: len keys at positions pos0 .. pos0 + len - 1 (pos0 = 0
        // but for the branches of a shared prefix), raw rows from its first row
        const int sq = p.tile_seg[blockIdx.x], pos0 = p.seg[4 * sq + 3];
        T = pos0 + p.seg[4 * sq];
        row_base = p.seg[4 * sq + 1] - pos0;
        t0 = pos0 + (tile - p.seg[4 * sq + 2]) * KT;
    }
    const size_t tile_off = ((size_t)c * (p.Tpad / KT) + tile) * (size_t)(KT * D);

    wk1[tid] = 1.0f + bf2f(p.wk[tid]);
    for (int it = 0; it < 4; ++it) {
        const int idx = it * 256 + tid, r = idx >> 5, ch = idx & 31, key = t0 + r;
        uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (key < T) {
            const size_t off = ((size_t)(key + row_base) * p.Hkv + c) * D + ch * 8;
            kv = *reinterpret_cast<const uint4 *>(p.k + off);
            vv = *reinterpret_cast<const uint4 *>(p.v + off);
        }
        *reinterpret_cast<uint4 *>(&ks[r][ch * 8]) = kv;
        *reinterpret_cast<uint4 *>(&vs[r][ch * 8]) = vv;
    }
    __syncthreads();

    if (tid < KT) {
        // Sum of squares of key row tid in ascending dimension order; the
        // row's 16-byte chunks are read from LDS eight ahead of the chain.
        const uint4 *row = reinterpret_cast<const uint4 *>(&ks[tid][0]);
        uint4 buf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            buf[i] = row[i];
        float ss = 0.0f;
#pragma unroll
        for (int ch = 0; ch < D / 8; ++ch) {
            const uint4 u = buf[ch & 7];
            if (ch + 8 < D / 8)
                buf[ch & 7] = row[ch + 8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = word_f(u, t);
                ss += x * x;
            }
        }
        rs[tid] = 1.0f / sqrtf(ss / (float)D + p.eps);
    } else if (tid >= 64) {
        // Meanwhile waves 1..3 store the transposed value tile, or encode the
        // fp8 value rows (512 row chunks over 192 threads; a row's 16 chunks
        // are 16 consecutive lanes of one wave).
        if (!FP8) {
            write_vt_tile(vs, p.vt + tile_off, tid - 64, 192);
        } else {
            for (int idx = tid - 64; idx < 32 * 16; idx += 192) {
                const int r = idx >> 4, ch = idx & 15;
                fp8_row_chunk(&vs[r][16 * ch], ch, t0 + r < T, p.v8 + ((size_t)c * p.Tpad + t0 + r) * D + 16 * ch,
                              p.v8s + (size_t)c * p.Tpad + t0 + r);
            }
        }
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
            n[s] = round_op((bf2f(ks[r][d]) * rr) * wk1[d]);
        }
        if (key < T) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int j = sub + 8 * s;
                const float cj = round_op(p.cos_tab[(size_t)key * HALF_R + j]);
                const float sj = round_op(p.sin_tab[(size_t)key * HALF_R + j]);
                const float a = n[s], b = n[s + 4];
                n[s] = round_op(round_op(a * cj) + round_op(-b * sj));
                n[s + 4] = round_op(round_op(b * cj) + round_op(a * sj));
            }
        }
#pragma unroll
        for (int s = 0; s < 32; ++s)
            ks[r][sub + 8 * s] = (key < T) ? f2bf(n[s]) : (uint16_t)0;
    }
    __syncthreads();

    if (!FP8) {
        write_k_tile(ks, p.kp + tile_off, tid);
        return;
    }
    // fp8 key rows (the value rows were encoded during the chain above).
    for (int it = 0; it < 2; ++it) {
        const int idx = it * 256 + tid, r = idx >> 4, ch = idx & 15;
        fp8_row_chunk(&ks[r][16 * ch], ch, t0 + r < T, p.k8 + ((size_t)c * p.Tpad + t0 + r) * D + 16 * ch,
                      p.k8s + (size_t)c * p.Tpad + t0 + r);
    }
}

// Widens fp8 cache rows 0..T-1 into the Kp / Vt tiles.  grid (tiles, Hkv).
__global__ __launch_bounds__(256) void kv_widen(KvWidenParams p)
{
    __shared__ __align__(16) uint16_t ks[KT][D + 8];
    __shared__ __align__(16) uint16_t vs[KT][D + 8];
    const int tile = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, t0 = tile * KT;
    for (int it = 0; it < 4; ++it) {
        const int idx = it * 256 + tid, isv = idx >> 9, r = (idx >> 4) & 31, ch = idx & 15;
        const int key = t0 + r;
        uint32_t o[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if (key < p.T) {
            const size_t row = (size_t)c * p.Tpad + key;
            const uint4 cw = *reinterpret_cast<const uint4 *>((isv ? p.v8 : p.k8) + row * D + 16 * ch);
            const float sc = (isv ? p.v8s : p.k8s)[row];
            const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
            // The hardware's e4m3 -> fp32 convert is exact; fp32 product,
            // one rounding to bf16.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const auto v01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[q], false);
                const auto v23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[q], true);
                o[2 * q] = pack2(v01[0] * sc, v01[1] * sc);
                o[2 * q + 1] = pack2(v23[0] * sc, v23[1] * sc);
            }
        }
        uint16_t *dst = isv ? &vs[r][16 * ch] : &ks[r][16 * ch];
        *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    __syncthreads();
    write_kv_tile(ks, vs, p.kp, p.vt, ((size_t)c * (p.Tpad / KT) + tile) * (size_t)(KT * D), tid);
}

#ifdef ATTN_TEST_HOOKS
// Debug: the fp8 cache writer's arithmetic for finite rows on single values:
// q[i] = x[i] / sc[i] (div_rn with y = 1 / sc[i]) and codes[i] = its e4m3
// code (enc4_e4m3).  One value per thread; grid ceil(n / 256).
__global__ __launch_bounds__(256) void fp8_encode_debug(const float *x, const float *sc, float *q, uint8_t *codes,
                                                        int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float s = sc[i];
    const float v = div_rn(x[i], s, 1.0f / s);
    q[i] = v;
    codes[i] = (uint8_t)(enc4_e4m3(v, 0.0f, 0.0f, 0.0f) & 0xffu);
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
#endif  // ATTN_TEST_HOOKS

// ---------------------------------------------------------------------------
// Mask packing (launch shape below).
// bits[w][row] bit b = mask[row][32w+b] != 0 && 32w+b <= row && 32w+b < S
// (key word major: a tile's words of consecutive rows are adjacent; rows
// S .. bstride-1 get zero words).
// tilevis[rb][w] = any bit of the 64 x 32 block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nz_bits4(uint32_t u)
{
    return ((u & 0x000000ffu) ? 1u : 0u) | ((u & 0x0000ff00u) ? 2u : 0u) |
           ((u & 0x00ff0000u) ? 4u : 0u) | ((u & 0xff000000u) ? 8u : 0u);
}

// grid (ceil(W / 32), row blocks of 64), 256 threads: thread t takes key
// word w0 + (t & 31) of the 8 rows 8 (t >> 5) .. +7 of the block, all eight
// rows' loads in flight at once; the 8 row groups' OR of the words gives the
// tile flag (through LDS).
__global__ __launch_bounds__(256) void mask_pack(MaskPackParams p)
{
    __shared__ uint32_t anyw[8][32];
    const int tid = threadIdx.x, wl = tid & 31, rg = tid >> 5;
    const int w = blockIdx.x * 32 + wl;
    const int rb = blockIdx.y;
    const int key0 = 32 * w;
    const int row0 = rb * QW + 8 * rg;
    uint32_t words[8];
    if (w < p.W && p.vec16 && key0 + 32 <= p.S) {
        uint4 a[8], b[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = row0 + r;
            a[r] = b[r] = make_uint4(0u, 0u, 0u, 0u);
            if (row < p.S && key0 <= row) {
                const uint8_t *src = p.mask + (size_t)row * p.S + key0;
                a[r] = *reinterpret_cast<const uint4 *>(src);
                b[r] = *reinterpret_cast<const uint4 *>(src + 16);
            }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
            words[r] = nz_bits4(a[r].x) | (nz_bits4(a[r].y) << 4) | (nz_bits4(a[r].z) << 8) |
                       (nz_bits4(a[r].w) << 12) | (nz_bits4(b[r].x) << 16) | (nz_bits4(b[r].y) << 20) |
                       (nz_bits4(b[r].z) << 24) | (nz_bits4(b[r].w) << 28);
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = row0 + r;
            uint32_t word = 0;
            if (w < p.W && row < p.S && key0 <= row) {
                const uint8_t *src = p.mask + (size_t)row * p.S + key0;
                for (int bit = 0; bit < 32; ++bit)
                    if (key0 + bit < p.S && src[bit] != 0)
                        word |= 1u << bit;
            }
            words[r] = word;
        }
    }
    uint32_t any = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int row = row0 + r;
        const int last = row - key0;                   // keys key0..row are causal
        if (last < 0)
            words[r] = 0;
        else if (last < 31)
            words[r] &= (2u << last) - 1u;
        any |= words[r];
    }
    // The 8 rows' words are adjacent in bits (row0 + 7 < bstride, 32-byte aligned).
    if (w < p.W) {
        uint4 *dst = reinterpret_cast<uint4 *>(p.bits + (size_t)w * p.bstride + row0);
        dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
        dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
    }
    anyw[rg][wl] = any;
    __syncthreads();
    if (rg == 0 && w < p.W) {
#pragma unroll
        for (int g = 1; g < 8; ++g)
            any |= anyw[g][wl];
        p.tilevis[(size_t)rb * p.W + w] = any ? 1 : 0;
    }
}

__device__ __forceinline__ void load_queries1(const AttnParams &p, int r0, int h, int lane, uint4 (&qf)[16],
                                              const float *wq1);

// (1 + w_q) in fp32 for the query prologue, in LDS; the caller's barrier
// publishes it.  Needs at least D threads.
__device__ __forceinline__ void fill_wq1(float *wq1, const uint16_t *wq)
{
    if (threadIdx.x < D)
        wq1[threadIdx.x] = 1.0f + bf2f(wq[threadIdx.x]);
}

#ifdef ATTN_TEST_HOOKS
// Debug: prepared queries in a plain [rows][Hq][D] layout.
// grid (ceil(S/64), ceil(Hq/4)), 256 threads: wave = one head, 64 rows.
__global__ __launch_bounds__(256) void q_prologue_debug(AttnParams p, uint16_t *qp)
{
    __shared__ __align__(16) float wq1[D];
    fill_wq1(wq1, p.wq);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y * 4 + wave;
    if (h >= p.Hq)
        return;
    const int r0 = blockIdx.x * 64;
    uint4 qf[2][16];
    load_queries1(p, r0, h, lane, qf[0], wq1);
    load_queries1(p, r0 + 32, h, lane, qf[1], wq1);
    const int j = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int row = r0 + 32 * b + j;
        if (row < p.S) {
#pragma unroll
            for (int c = 0; c < 16; ++c)
                *reinterpret_cast<uint4 *>(qp + ((size_t)row * p.Hq + h) * D + 16 * c + 8 * hh) = qf[b][c];
        }
    }
}
#endif  // ATTN_TEST_HOOKS

// ---------------------------------------------------------------------------
// Attention helpers.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int QB = 32;                   // query rows per MFMA block (one per wave)
constexpr int MAX_TILES = 32768 / KT;    // tile list capacity (token cap / 32)
constexpr int TILE_BYTES = KT * D * 2;   // one K or V^T tile: 16 KB
constexpr int EP_STRIDE = 2 * D + 16;    // epilogue staging: bytes per row

// Global -> LDS copies (global_load_lds_dwordx4 / _dword).  The instruction
// reads gbase + voff + OFF per lane and writes LDS at M0 + OFF + 16 L (4 L for
// the dword form) for lane L: the immediate offset applies to both addresses,
// so the parts of one tile share M0, the base and the lane offset.  gbase and
// m0 must be wave-uniform.  M0 is an operand, so the compiler writes it and
// knows it is in use; a copy right after an M0 write needs one wait state,
// which the first copy after a new M0 value (NOP) supplies.  Issued through
// inline asm so the compiler does not guard later LDS reads of *other*
// buffers with a wait on these loads; the caller orders them with an explicit
// s_waitcnt vmcnt before the barrier that publishes the buffer.
template <int OFF, bool NOP>
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t m0)
{
    if (NOP)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2"
                     :: "v"(voff), "s"(gbase), "i"(OFF), "{m0}"(m0) : "memory");
    else
        asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2"
                     :: "v"(voff), "s"(gbase), "i"(OFF), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void *gbase, uint32_t voff, uint32_t m0)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" :: "v"(voff), "s"(gbase), "{m0}"(m0) : "memory");
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

// ---------------------------------------------------------------------------
// Context accumulators.  O^T of a wave's 32-row block is 8 groups of (32 dims
// x 32 queries) fp32 = the wave's 128 AGPRs; the VGPRs hold the queries,
// scores and weights.  The context MFMAs are inline asm with AGPR
// accumulators.  The compiler does not track their latency, so the software
// wait states the ISA requires around them are inserted here: VALU access to
// an accumulator waits (up to 19 states) for the last MFMA on it, and each
// MFMA waits (a few states) for weights a VALU may have just written.  Taking
// the accumulators as operands keeps the nops between the two.
// ---------------------------------------------------------------------------
// The weights operand b is VALU-written.  Where that write may be close
// before (the first MFMA on each operand word) a leading nop covers the
// dependency; the build checks every inline MFMA's operands in the final code.
template <bool NOP>
__device__ __forceinline__ void mfma_o(f32x16 &acc, const bf16x8 &a, const u32x4 &b)
{
    if (NOP)
        asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void acc_wait(f32x16 (&o)[8])
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                   "+a"(o[7]));
}


// ---------------------------------------------------------------------------
// Online softmax of one block's tile as a program of 32 steps placed between
// MFMAs.  A step holds a few VALU instructions, none depending on another of
// the same step, so the matrix pipe does not wait on them.
//   lane (j, hh) holds query j and keys 8g + 4hh + r of the tile (e = 4g + r).
//   steps 0..7  : tile max (a tree of max3 on the fp32 scores, then the
//                 partner lane's max for the tile's other 16 keys; rounding is
//                 monotonic, so rounding the max afterwards gives the max of
//                 the rounded scores); the scores rounded to bf16 in place;
//   steps 8..13 : running max (moved only past the threshold), alpha, base;
//   steps 12..29: weights p = exp2(x log2(e)/16 - base), two per pair of
//                 steps, packed to the bf16 MFMA operand; the row sum adds the
//                 packed bf16 weights (the values the context product uses);
//   steps 30, 31: l = l alpha + sum.
// Masked path: 8 steps before these hide the scores of invisible keys.
// ---------------------------------------------------------------------------
constexpr int HIDE_STEPS = 8;
constexpr uint32_t BF16_ONES = 0x3f803f80u;     // (1.0, 1.0) as packed bf16

// Materialises a value at this point of the instruction stream (the
// compiler would otherwise sink the softmax arithmetic past the rescale
// branch to its first use, out of the MFMA gaps it was placed in).
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

// The softmax steps use these opaque forms so that the compiler keeps them
// as written (it would otherwise quieten NaNs before each max, and split a
// packed rounding into two single ones when only unpacked halves are used).
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2f(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t pack2_op(float a, float b)
{
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}


__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

struct SmTmp {
    float a, b, c, d, e, f, g, mt, mt2, t1, mn, dd, bn, nb, ar, L0, L1;
    bool up, minf, same, ninf;
};

__device__ __forceinline__ void hide_step(int i, f32x16 &s, uint32_t vh)
{
#pragma unroll
    for (int e = 2 * i; e < 2 * i + 2; ++e) {
        const int sh = 8 * (e >> 2) + (e & 3);
        const uint32_t keep = (uint32_t)((int32_t)(vh << (31 - sh)) >> 31);
        s[e] = __uint_as_float((__float_as_uint(s[e]) & keep) | (0xff800000u & ~keep));
    }
}

__device__ __forceinline__ void hide_all(f32x16 &s, uint32_t vh)
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        hide_step(i, s, vh);
}

// Weight pair q: F = the two exponent arguments, E = the two exp2, C = pack
// to bf16 (the MFMA operand word), D = add the pair to a partial row sum.
__device__ __forceinline__ void sm_pair_F(int q, f32x16 &s, const SmTmp &t)
{
    s[2 * q] = __builtin_fmaf(s[2 * q], SCALE_LOG2, t.nb);
    s[2 * q + 1] = __builtin_fmaf(s[2 * q + 1], SCALE_LOG2, t.nb);
}
__device__ __forceinline__ void sm_pair_E(int q, f32x16 &s)
{
    s[2 * q] = __builtin_amdgcn_exp2f(s[2 * q]);
    s[2 * q + 1] = __builtin_amdgcn_exp2f(s[2 * q + 1]);
}
__device__ __forceinline__ void sm_pair_C(int q, const f32x16 &s, u32x4 (&pw)[2])
{
    const uint32_t pq = pack2_op(s[2 * q], s[2 * q + 1]);
    pw[q >> 2][q & 3] = pq;
}
__device__ __forceinline__ void sm_pair_D(int q, const u32x4 (&pw)[2], SmTmp &t)
{
    const uint32_t pq = pw[q >> 2][q & 3];
    if (q & 1)
        t.L1 = dot2_bf16(pq, BF16_ONES, q == 1 ? 0.0f : t.L1);
    else
        t.L0 = dot2_bf16(pq, BF16_ONES, q == 0 ? 0.0f : t.L0);
}

__device__ __forceinline__ void sm_step(int i, f32x16 &s, float &m, float &l, float &alpha, u32x4 (&pw)[2],
                                        SmTmp &t)
{
    if (i == 0) {
        t.a = max3f(s[0], s[1], s[2]);
        t.b = max3f(s[3], s[4], s[5]);
        t.c = max3f(s[6], s[7], s[8]);
        t.d = max3f(s[9], s[10], s[11]);
    } else if (i == 1) {
        t.e = max3f(s[12], s[13], s[14]);
        s[0] = round_op(s[0]);
        s[1] = round_op(s[1]);
        s[2] = round_op(s[2]);
    } else if (i == 2) {
        t.f = max3f(t.a, t.b, t.c);
        t.g = max3f(t.d, t.e, s[15]);
        s[3] = round_op(s[3]);
        s[4] = round_op(s[4]);
    } else if (i == 3) {
        t.mt = max2f(t.f, t.g);
        s[5] = round_op(s[5]);
        s[6] = round_op(s[6]);
        s[7] = round_op(s[7]);
    } else if (i == 4) {
        // Partner lane's max: v_permlane32_swap fed the value twice leaves
        // this lane's and the partner's value in the two results.
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t.mt), __float_as_uint(t.mt), false, false);
        t.mt = __uint_as_float(r[0]);
        t.mt2 = __uint_as_float(r[1]);
        t.t1 = m + TAU_X;
        s[8] = round_op(s[8]);
    } else if (i == 5) {
        t.mt = max2f(t.mt, t.mt2);
        s[9] = round_op(s[9]);
        s[10] = round_op(s[10]);
        s[11] = round_op(s[11]);
    } else if (i == 6) {
        t.mt = round_op(t.mt);                  // bf16-rounded tile max
        s[12] = round_op(s[12]);
        s[13] = round_op(s[13]);
        s[14] = round_op(s[14]);
    } else if (i == 7) {
        s[15] = round_op(s[15]);
    } else if (i == 8) {
        t.up = t.mt > t.t1;
        t.minf = (m == -INFINITY);
    } else if (i == 9) {
        t.mn = t.up ? t.mt : m;
    } else if (i == 10) {
        t.dd = m - t.mn;
        t.same = (t.mn == m);
        t.bn = t.mn * -SCALE_LOG2;
        t.ninf = (t.mn == -INFINITY);
    } else if (i == 11) {
        t.dd = t.dd * SCALE_LOG2;
        t.nb = t.ninf ? 0.0f : t.bn;            // a finite base while nothing is visible
    } else if (i == 12) {
        t.ar = __builtin_amdgcn_exp2f(t.dd);
        sm_pair_F(0, s, t);
    } else if (i == 13) {
        // While nothing was visible (m = -inf) O and l are zero: no rescale.
        alpha = (t.same || t.minf) ? 1.0f : t.ar;
        pin(alpha);
        m = t.mn;
        sm_pair_E(0, s);
    } else if (i < 28) {
        // 14, 16, .., 26: F(q+1), C(q) for q = (i-14)/2;  15, .., 27: E(q+1), D(q).
        const int q = (i - 14) >> 1;
        if ((i & 1) == 0) {
            sm_pair_F(q + 1, s, t);
            sm_pair_C(q, s, pw);
        } else {
            sm_pair_E(q + 1, s);
            sm_pair_D(q, pw, t);
        }
    } else if (i == 28) {
        sm_pair_C(7, s, pw);
    } else if (i == 29) {
        sm_pair_D(7, pw, t);
    } else if (i == 30) {
        t.L0 = t.L0 + t.L1;
    } else if (i == 31) {
        l = __builtin_fmaf(l, alpha, t.L0);
        pin(l);
    }
}

__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>((uintptr_t)addr);
}

__device__ __forceinline__ void rescale(f32x16 (&o)[8], float alpha)
{
    if (__builtin_expect(__any(alpha != 1.0f), 0)) {
        acc_wait(o);
        // In place in the AGPRs (a VGPR round trip visible to the compiler
        // would make it keep the accumulators in VGPRs across the branch).
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = o[db][e];
                float tmp;
                asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                             : "+a"(x), "=&v"(tmp)
                             : "v"(alpha));
                o[db][e] = x;
            }
        acc_wait(o);
    }
}

// ---------------------------------------------------------------------------
// Attention.  A work item is 64 query rows x the 4 query heads of a head
// group of one KV head (the K/V tiles it stages serve all four heads), on 8
// waves, two per SIMD: wave w owns head 4hg + (w & 3) and
// the 32-row block w >> 2, so a SIMD holds the two blocks of one head.  A
// wave's registers (at most 256 with two waves per SIMD) hold one block: O
// (128 AGPRs), its query fragments (64) and the scores of one tile (16).  The
// issue port of a SIMD is shared by its two waves, which roughly doubles the
// instruction budget around each MFMA compared with one wave per SIMD.  The
// two blocks run complementary phases of the same key interval:
//   block 0, interval k: [S(k)]                 [O += V(k-1) P(k-1) | softmax k  ]
//   block 1, interval k: [O += V(k-2) P(k-2) | softmax k-1]  [S(k)]
// so while one wave issues the softmax's vector work the other issues a run
// of plain MFMAs.  Each wave moves an eighth of every K and V^T tile into
// LDS (2 KB), K three tiles ahead and V^T two ahead, four buffers
// each (block 1 still reads V(k-2) while V(k+1) arrives).
// MASKED: the walk follows the tiles with a visible key for some row of the
// 64 (from mask_pack's flags); each tile's 64 visibility words are copied to
// LDS next to its K tile, and the softmax program starts with 8 steps that
// hide invisible keys.  BIDIR: no causal predicate (every row walks all key
// tiles; only keys past T are hidden).
// ---------------------------------------------------------------------------
constexpr int ATHREADS8 = 512;
constexpr int SMEM8 = (8 * TILE_BYTES > 8 * QB * EP_STRIDE) ? 8 * TILE_BYTES : 8 * QB * EP_STRIDE;

// Query prologue of one 32-row block (rows r0 .. r0+31) of head h: loads the
// q half of the rows, applies (1+w) RMSNorm (sum of squares in ascending
// dimension order, the same chain as the key prologue) and partial RoPE, and
// leaves the MFMA B-operand fragments in qf[c]: lane (j = lane & 31, hh =
// lane >> 5) holds dims 16c + 8hh .. +7 of row r0 + j.  Rows at or past S are
// zero.  wq1 is (1 + w_q) in fp32, in LDS (the same fp32 sum the plain
// definition forms per element).
// The sum of squares runs on the lanes that hold the first 8 dims of each
// 16-dim chunk (hh = 0): each takes its partner lane's 8 (lane ^ 32, through
// ds_bpermute, which leaves the fragments in place) and chains the 16 in
// dimension order.  The hh = 1 lanes run the same instructions on the two
// halves swapped and then take their partner's sum, so both lanes of a row
// hold the one ascending chain.
__device__ __forceinline__ void load_queries1(const AttnParams &p, int r0, int h, int lane, uint4 (&qf)[16],
                                              const float *wq1)
{
    const int j = lane & 31, hh = lane >> 5;
    const int row = r0 + j;
    const bool ok = row < p.S;
    const uint16_t *src = p.qg + (((size_t)(ok ? row : 0) * p.Hq + h) * 2) * D;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        qf[c] = *reinterpret_cast<const uint4 *>(src + 16 * c + 8 * hh);
    const int partner = (lane ^ 32) << 2;
    auto one = [&](uint32_t w) { return (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)w); };
    auto from_partner = [&](const uint4 &u) { return make_uint4(one(u.x), one(u.y), one(u.z), one(u.w)); };
    float ss = 0.0f;
    // The partner's words are fetched one chunk ahead (the fences keep the
    // compiler from fetching them all up front, which would hold 64 more
    // registers).
    uint4 other = from_partner(qf[0]);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        uint4 next = other;
        if (c + 1 < 16)
            next = from_partner(qf[c + 1]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float x = word_f(qf[c], t);
            ss += x * x;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float x = word_f(other, t);
            ss += x * x;
        }
        __builtin_amdgcn_sched_barrier(0);
        other = next;
    }
    {
        // lanes hh = 1 take the chain of lane (j, 0): the first result of a
        // swap fed the same value twice is the lower-half lane's value.
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(r[0]);
    }
    const float rr = 1.0f / sqrtf(ss / (float)D + p.eps);
    // (1 + w) of a chunk's 8 dims, read one chunk ahead (fenced like the
    // partner words above).
    struct W8 {
        float4 a, b;
        __device__ float operator[](int t) const
        {
            return t == 0 ? a.x : t == 1 ? a.y : t == 2 ? a.z : t == 3 ? a.w
                 : t == 4 ? b.x : t == 5 ? b.y : t == 6 ? b.z : b.w;
        }
    };
    auto w_of = [&](int c) {
        return W8{*reinterpret_cast<const float4 *>(wq1 + 16 * c + 8 * hh),
                  *reinterpret_cast<const float4 *>(wq1 + 16 * c + 8 * hh + 4)};
    };
    // The norm unpacks the fragment words again: hidden from the compiler,
    // which would otherwise keep the chain's 128 unpacked values alive until
    // here (more registers than a wave has).
    auto fresh = [](const uint4 &u) {
        u32x4 v = {u.x, u.y, u.z, u.w};
        asm volatile("" : "+v"(v));
        return make_uint4(v[0], v[1], v[2], v[3]);
    };
    W8 wv = w_of(4);
#pragma unroll
    for (int c = 4; c < 16; ++c) {
        const W8 wn = w_of(c + 1 < 16 ? c + 1 : 0);
        const uint4 qv = fresh(qf[c]);
        float n[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            n[t] = (word_f(qv, t) * rr) * wv[t];
        qf[c] = make_uint4(pack2(n[0], n[1]), pack2(n[2], n[3]), pack2(n[4], n[5]), pack2(n[6], n[7]));
        __builtin_amdgcn_sched_barrier(0);
        wv = wn;
    }
    // Rotary dims 0..63: chunks c and c + 2 hold the pairs (d, d + 32).
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
        const W8 wa = w_of(c), wb = w_of(c + 2);
        const uint4 qa = fresh(qf[c]), qb = fresh(qf[c + 2]);
        float a[8], b[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            a[t] = round_op((word_f(qa, t) * rr) * wa[t]);
            b[t] = round_op((word_f(qb, t) * rr) * wb[t]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float cj = round_op(cv[t]), sj = round_op(sv[t]);
            const float av = a[t], bv = b[t];
            a[t] = round_op(round_op(av * cj) + round_op(-bv * sj));
            b[t] = round_op(round_op(bv * cj) + round_op(av * sj));
        }
        qf[c] = make_uint4(pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(a[4], a[5]), pack2(a[6], a[7]));
        qf[c + 2] = make_uint4(pack2(b[0], b[1]), pack2(b[2], b[3]), pack2(b[4], b[5]), pack2(b[6], b[7]));
        __builtin_amdgcn_sched_barrier(0);
    }
    if (!ok) {
#pragma unroll
        for (int c = 0; c < 16; ++c)
            qf[c] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Scores half (one block): S^T(k) = K(k) . Q^T, 16 MFMAs, one per slot, K
// fragments read one ahead (the registers of a wave at two waves per SIMD
// allow no more); issue(slot) places the copies among the MFMAs.
template <typename Issue>
__device__ __forceinline__ void s_half8(uint32_t kaddr, const uint4 (&qf)[16], f32x16 &s, Issue &&issue)
{
    bf16x8 kf[16];
    // The wave in its scores half issues first when both waves of the SIMD
    // have an instruction ready (its MFMA stream keeps the matrix pipe fed
    // while the other wave's context half interleaves the softmax); the
    // context half drops back to the base level.
    asm volatile("s_setprio 1");
    kf[0] = lds_read16(kaddr);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        if (c + 1 < 16)
            kf[c + 1] = lds_read16(kaddr + 1024 * (c + 1));
        const f32x16 z = {};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], __builtin_bit_cast(bf16x8, qf[c]), c ? s : z, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue(c);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Softmax step i of the one-block program.  The packs of weight pairs 4..7
// (the second operand word group) and the row-sum tail are left to
// sm_tail8: the context MFMAs of the same half still read that group.
__device__ __forceinline__ void sm_step8(int i, f32x16 &s, float &m, float &l, float &alpha, u32x4 (&pw)[2],
                                         SmTmp &t)
{
    if (i >= 14 && i < 28) {
        const int q = (i - 14) >> 1;
        if ((i & 1) == 0) {
            sm_pair_F(q + 1, s, t);
            if (q < 4)
                sm_pair_C(q, s, pw);
        } else {
            sm_pair_E(q + 1, s);
            if (q < 4)
                sm_pair_D(q, pw, t);
        }
    } else if (i < 14) {
        sm_step(i, s, m, l, alpha, pw, t);
    }
}
__device__ __forceinline__ void sm_tail8(f32x16 &s, float &l, float alpha, u32x4 (&pw)[2], SmTmp &t)
{
#pragma unroll
    for (int q = 4; q < 8; ++q)
        sm_pair_C(q, s, pw);
#pragma unroll
    for (int q = 4; q < 8; ++q)
        sm_pair_D(q, pw, t);
    t.L0 = t.L0 + t.L1;
    l = __builtin_fmaf(l, alpha, t.L0);
    pin(l);
}

// Context half (one block): O^T += V^T . P^T for the tile whose weights are
// in pw (16 MFMAs, kc-major: the first 8 read only the first operand word
// group; V fragments read one ahead), with the softmax of the scores s in the
// gaps, two steps per slot from slot 1 (the last score MFMA may still be in
// flight at slot 0).  The first word group is repacked only after the eighth
// MFMA and the second after the last, so one weight buffer serves both tiles.
template <bool MASKED, bool DO_PV, bool DO_SM>
__device__ __forceinline__ void pv_half8(uint32_t vaddr, f32x16 (&o)[8], u32x4 (&pw)[2], f32x16 &s, float &m,
                                         float &l, float &alpha, uint32_t vh)
{
    SmTmp t;
    bf16x8 vf[16];
    asm volatile("s_setprio 0");
    if (DO_PV)
        vf[0] = lds_read16(vaddr);
    // Masked: the 8 hide steps come first; the program then runs past the
    // 16 MFMA slots (the other wave of the SIMD keeps the matrix pipe busy).
    constexpr int NSLOT = (DO_SM && MASKED) ? 19 : 16;
    auto step = [&](int x) {
        if (MASKED) {
            if (x < HIDE_STEPS)
                hide_step(x, s, vh);
            else
                sm_step8(x - HIDE_STEPS, s, m, l, alpha, pw, t);
        } else {
            sm_step8(x, s, m, l, alpha, pw, t);
        }
    };
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
        if (DO_PV && i < 16) {
            if (i + 1 < 16) {
                const int n1 = i + 1;
                vf[n1] = lds_read16(vaddr + 8192 * (n1 >> 3) + 512 * (n1 & 7));
            }
            if ((i & 7) == 0)
                mfma_o<true>(o[i & 7], vf[i], pw[i >> 3]);
            else
                mfma_o<false>(o[i & 7], vf[i], pw[i >> 3]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (DO_SM && i >= 1) {
            // The softmax reads s first through inline asm, for which the
            // compiler inserts no wait states after the last score MFMA (the
            // compiler's own); these complete the count on every path into
            // this slot (the first tile has no context MFMAs before it).
            if (i == 1 && DO_PV)
                asm volatile("s_nop 4");
            else if (i == 1)
                asm volatile("s_nop 7\n\ts_nop 7");
            step(2 * i - 2);
            step(2 * i - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (DO_SM)
        sm_tail8(s, l, alpha, pw, t);
}

// The attention pass.  SHARED: a packed batch of branches that continue one
// shared prefix (key tiles below the prefix's length come from the caller's
// cache, the branch's own tiles from the workspace, positions from the
// prefix's length on).
template <bool MASKED, bool BIDIR, bool SHARED>
__global__ __attribute__((amdgpu_flat_work_group_size(ATHREADS8, ATHREADS8), amdgpu_waves_per_eu(2, 2)))
void attn_fwd8(AttnParams pk)
{
    __shared__ __align__(16) char smem[SMEM8];     // K tiles 0..3, V^T tiles 4..7; epilogue staging
    __shared__ uint32_t bitsbuf[MASKED ? 8 : 1][QW];
    __shared__ int tile_list[MASKED ? MAX_TILES : 1];
    __shared__ int tile_count;
    __shared__ __align__(16) float wq1[D];

    const int lane_id = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hw = wave & 3;                        // head within the group of four
    const int blk = wave >> 2;                      // 32-row block; 1 = the lagging phase

    // Work items (64-row block, KV head, head group), row blocks heaviest
    // first (longest key walk; a packed batch lists its (sequence, row block)
    // pairs in that order), are dealt to at most one workgroup per compute
    // unit by sched_item: a snake order, KV heads kept to their own XCDs.
    const int P = (int)gridDim.x;
    fill_wq1(wq1, pk.wq);
    __syncthreads();
#pragma clang loop unroll(disable)
    for (int pass = 0;; ++pass) {
        SchedItem si;
        if (pk.sched) {
            // (uniform values: the workgroup's own table entries)
            const int o = __builtin_amdgcn_readfirstlane(pk.sched[blockIdx.x]) + pass;
            if (o >= __builtin_amdgcn_readfirstlane(pk.sched[blockIdx.x + 1]))
                break;
            si = sched_unpack(__builtin_amdgcn_readfirstlane(pk.sched[P + 1 + o]));
        } else if (!sched_item((int)blockIdx.x, P, pass, pk.nrb, pk.Hkv, pk.n_hg, si)) {
            break;
        }
        if (pass > 0)
            __syncthreads();                         // the previous item is done with LDS
        // The lane index, rebuilt every pass by instructions the compiler
        // cannot hoist (kept across the whole loop it would hold a register
        // through the key walk, and the walk has none to spare).
        int lane;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
        const int j = lane & 31, hh = lane >> 5;
        // The item's problem: the launch's, or one sequence of a packed batch
        // (its rows, its prepared key tiles, positions from 0).
        AttnParams p = pk;
        int rb, ktile0 = 0, ptiles = 0;
        if (SHARED || (!BIDIR && !MASKED && pk.pairs)) {
            const int sq = pk.pairs[2 * si.rbi];
            rb = pk.pairs[2 * si.rbi + 1];
            p.S = p.T = pk.seg[4 * sq];
            p.q_base = 0;
            p.qg = pk.qg + (size_t)pk.seg[4 * sq + 1] * pk.Hq * 2 * D;
            p.out = pk.out + (size_t)pk.seg[4 * sq + 1] * pk.Hq * D;
            ktile0 = pk.seg[4 * sq + 2];
            if (SHARED) {
                // A branch: query positions and keys continue from the prefix.
                const int pos0 = __builtin_amdgcn_readfirstlane(pk.seg[4 * sq + 3]);
                p.T += pos0;
                p.q_base = pos0;
                ptiles = pos0 / KT;
            }
        } else {
            rb = pk.nrb - 1 - si.rbi;
        }
        const int kvh = si.kvh, hg = si.hg;
        const int gidx = hg * 4 + hw;
        const bool active = gidx < p.G;
        const int h = kvh * p.G + (active ? gidx : 0);
        const int r0 = rb * QW;
        // A split item (half 1 or 2, causal or masked launches with fewer
        // items than compute units) computes one 32-row block on waves 0..3 alone;
        // waves 4..7 then only copy their parts of the tiles and keep the
        // barrier count.  A row's arithmetic is the same either way.
        const int half = si.half;
        const bool idle = half != 0 && blk == 1;
        const int bq = half != 0 ? half - 1 : blk;       // this wave's 32-row block of the 64
        const int rbase = r0 + QB * bq;                  // this wave's rows rbase .. rbase + 31

        const int P0 = p.q_base + r0;
        const int last_row = P0 + (half == 1 ? QB - 1 : QW - 1);
        const int ntiles = BIDIR ? (p.T + KT - 1) / KT : min(last_row, p.T - 1) / KT + 1;
        const int diag = P0 / KT + bq;                   // this block's diagonal tile

        // The walk: every tile up to the diagonal (>= 1: row r0 sees key 0), or
        // (masked) the tiles with a visible key for some row of the 64, ascending.
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
        // Masked: 64 consecutive walk entries from entry wbase on (clamped to
        // the last), one per lane; the walk takes its tile numbers from this
        // register by lane index rather than through an LDS read and wait.
        // In interval k the walk needs entries k+1 .. k+3, and wbase is moved
        // to k+1 whenever k+1 is a multiple of 32, so they stay inside it.
        int walk_win = 0, wbase = 0;
        auto walk_window = [&](int base) {
            if (MASKED) {
                wbase = base;
                walk_win = tile_list[min(base + lane, n - 1)];
            }
        };

        const uint32_t smem_base = lds_addr(smem);
        const uint16_t *kbase = p.kp + ((size_t)kvh * (p.Tpad / KT) + ktile0) * (KT * D);
        const uint16_t *vbase = p.vt + ((size_t)kvh * (p.Tpad / KT) + ktile0) * (KT * D);
        // Wave w moves bytes [2048 w, 2048 w + 2048) of every tile, in two parts.
        const uint32_t voff = (uint32_t)(wave * 2048 + lane * 16);
        auto m0_of = [&](bool is_k, int u) {
            return (uint32_t)__builtin_amdgcn_readfirstlane(
                (int)(smem_base + TILE_BYTES * ((is_k ? 0 : 4) + (u & 3)) + wave * 2048));
        };
        // (a branch's tiles below ptiles are the shared prefix's, in the cache)
        const uint16_t *ckbase = SHARED ? pk.ckp + (size_t)kvh * (p.Tpad / KT) * (KT * D) : nullptr;
        const uint16_t *cvbase = SHARED ? pk.cvt + (size_t)kvh * (p.Tpad / KT) * (KT * D) : nullptr;
        auto src_of = [&](bool is_k, int tile) {
            tile = __builtin_amdgcn_readfirstlane(tile);
            if (SHARED) {
                if (tile < ptiles)
                    return (is_k ? ckbase : cvbase) + (size_t)tile * (KT * D);
                tile -= ptiles;
            }
            return (is_k ? kbase : vbase) + (size_t)tile * (KT * D);
        };
        auto tile_clamped = [&](int u) -> int {
            return MASKED ? __builtin_amdgcn_readlane(walk_win, u - wbase) : min(u, n - 1);
        };
        // Masked: the 64 rows' visibility words of a tile, next to its K copy;
        // wave w moves the words of rows 8w .. 8w+7 (lane L writes word L),
        // 32 adjacent bytes of the key-word-major bits.
        const uint32_t bits_base = lds_addr(bitsbuf);
        auto load_bits = [&](int tile, int slot) {
            if (MASKED) {
                tile = __builtin_amdgcn_readfirstlane(tile);
                if ((lane >> 3) == wave) {
                    const int row = r0 + lane;                  // < bstride (pad rows hold zero words)
                    dma4(p.bits, (uint32_t)(((size_t)tile * p.bstride + row) * 4), bits_base + (uint32_t)(slot * QW * 4));
                }
            }
        };
        auto load_tile = [&](bool is_k, int u) {
            const uint16_t *src = src_of(is_k, tile_clamped(u));
            const uint32_t m0 = m0_of(is_k, u);
            dma16<0, true>(src, voff, m0);
            dma16<1024, MASKED>(src, voff, m0);
        };
        // Interval k's copies (issued in the wave's scores half): K(k+3) and
        // V(k+1), two parts each.
        auto issue_loads = [&](int k) {
            return [&, k](int slot) {
                if (slot == 1 || slot == 5) {
                    const uint16_t *src = src_of(true, tile_clamped(k + 3));
                    const uint32_t m0 = m0_of(true, k + 3);
                    if (slot == 1)
                        dma16<0, true>(src, voff, m0);
                    else
                        dma16<1024, MASKED>(src, voff, m0);
                } else if (slot == 9 || slot == 13) {
                    const uint16_t *src = src_of(false, tile_clamped(k + 1));
                    const uint32_t m0 = m0_of(false, k + 1);
                    if (slot == 9)
                        dma16<0, true>(src, voff, m0);
                    else
                        dma16<1024, MASKED>(src, voff, m0);
                } else if (MASKED && slot == 3) {
                    load_bits(tile_clamped(k + 3), (k + 3) & 7);
                }
            };
        };
        // Wait for the previous interval's copies (this interval's four, five
        // with the mask words, stay in flight), then the barrier.
        auto close_interval = [&]() {
            if (MASKED)
                asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            __syncthreads();
        };

        if (!MASKED || n > 0) {
            walk_window(0);
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                load_tile(true, u);
                load_bits(tile_clamped(u), u);
            }
            load_tile(false, 0);
        }

        if (idle) {
            // The other block's waves of a split item: their parts of every
            // copy (and of the mask words), the walk window, and the computing
            // waves' barriers: the prologue's; with a walk, one per interval and
            // one after the last context half; the epilogue's.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (!MASKED || n > 0) {
#pragma clang loop unroll(disable)
                for (int k = 0; k < n; ++k) {
                    if (MASKED && ((k + 1) & 31) == 0)
                        walk_window(k + 1);
                    auto iss = issue_loads(k);
                    iss(1);
                    iss(3);
                    iss(5);
                    iss(9);
                    iss(13);
                    close_interval();
                }
                close_interval();
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            continue;
        }

        uint4 qf[16];
        load_queries1(p, rbase, h, lane, qf, wq1);
        const FragOffsets fo = frag_offsets(j, hh);
        const uint32_t diag_vis = (j == 31) ? 0xffffffffu : ((2u << j) - 1u);

        f32x16 o[8];
        {
            uint32_t z;
            asm volatile("v_mov_b32 %0, 0" : "=v"(z));    // built here, not kept across passes
            const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{z, z, z, z});
#pragma unroll
            for (int db = 0; db < 8; ++db)
                asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(o[db]) : "v"(zero));
        }
        float m = -INFINITY, l = 0.0f, alpha = 1.0f;
        // Scores and weights need no initial value: the first score MFMA of
        // a tile takes a zero accumulator, and the first tile's softmax writes
        // all eight weight words before a context MFMA reads them.
        f32x16 s;
        u32x4 pw[2];

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        // Visibility of walk tile u for this block, as this lane's bits >> 4hh.
        auto masked_vh = [&](int u) -> uint32_t {
            return MASKED ? (bitsbuf[u & 7][QB * bq + j] >> (4 * hh)) : 0u;
        };
        auto causal_hide = [&](int u, f32x16 &sc) {
            if (MASKED) {
                // causality is folded into the mask words
            } else if (BIDIR) {
                if (u == n - 1 && (p.T & (KT - 1)) != 0)
                    hide_all(sc, ((1u << (p.T & (KT - 1))) - 1u) >> (4 * hh));
            } else if (u >= diag) {
                const uint32_t vis = (u == diag) ? diag_vis : 0u;
                hide_all(sc, vis >> (4 * hh));
            }
        };
        auto kaddr_of = [&](int k) {
            uint32_t a = smem_base + TILE_BYTES * (k & 3) + fo.k;
            asm volatile("" : "+v"(a));
            return a;
        };
        auto vaddr_of = [&](int k) {
            uint32_t a = smem_base + TILE_BYTES * (4 + (k & 3)) + fo.v;
            asm volatile("" : "+v"(a));
            return a;
        };
        const int cc = lane & 31;                       // epilogue: 16-byte chunk of a row
        uint4 gw[16];
        auto load_gates = [&]() {
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int row = min(rbase + 2 * it + hh, p.S - 1);
                gw[it] = *reinterpret_cast<const uint4 *>(p.qg + (((size_t)row * p.Hq + h) * 2 + 1) * D + 8 * cc);
            }
        };

        // Epilogue: ctx = bf16(O / l), out = bf16(ctx * bf16(sigmoid(gate))),
        // through LDS as whole 512-byte rows.
        auto epilogue = [&]() {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();                             // all waves are done with the tile buffers
            char *ep = smem + wave * QB * EP_STRIDE;
            const float lt = pair_sum(l);
            if (p.ml && hh == 0 && active && rbase + j < p.S) {
                p.ml[((size_t)(rbase + j) * p.Hq + h) * 2] = m;
                p.ml[((size_t)(rbase + j) * p.Hq + h) * 2 + 1] = lt;
            }
            const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
            acc_wait(o);
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = 32 * db + 8 * g + 4 * hh;
                    const uint2 cw = make_uint2(pack2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                                pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
                    *reinterpret_cast<uint2 *>(ep + j * EP_STRIDE + 2 * d0) = cw;
                }
            // Row rbase + 2 it + hh of the block: its staged context and its
            // output row, stepped by two rows per iteration.
            const char *crow = ep + hh * EP_STRIDE + 16 * cc;
            uint16_t *orow = p.out + ((size_t)(rbase + hh) * p.Hq + h) * D + 8 * cc;
            const size_t ostep = (size_t)2 * p.Hq * D;
            const int rows_left = active ? p.S - rbase - hh : 0;   // this lane stores iterations it < ceil(rows_left / 2)
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const uint4 cv = *reinterpret_cast<const uint4 *>(crow + 2 * it * EP_STRIDE);
                const uint32_t cws[4] = {cv.x, cv.y, cv.z, cv.w};
                const uint32_t gws[4] = {gw[it].x, gw[it].y, gw[it].z, gw[it].w};
                uint32_t ow[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float ov[2];
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const float ctx = hf ? hi_f(cws[q]) : lo_f(cws[q]);
                        const float gv = hf ? hi_f(gws[q]) : lo_f(gws[q]);
                        const float sg = round_op(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv * LOG2E)));
                        ov[hf] = ctx * sg;
                    }
                    ow[q] = pack2(ov[0], ov[1]);
                }
                if (2 * it < rows_left)
                    *reinterpret_cast<uint4 *>(orow) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
                orow += ostep;
            }
        };

        // Both phases run the same sequence S(0), softmax(0), S(1), O += V(0)P(0)
        // and softmax(1), ...; block 0 closes each interval after its context
        // half, block 1 after its scores half, which puts block 1 half an
        // interval behind.  The barrier is the workgroup's: each wave arrives
        // once per interval, from either place.
        const bool lag = blk == 1;
        if (!MASKED || n > 0) {
            s_half8(kaddr_of(0), qf, s, issue_loads(0));
            if (lag)
                close_interval();
            causal_hide(0, s);
            pv_half8<MASKED, false, true>(0u, o, pw, s, m, l, alpha, masked_vh(0));
            rescale(o, alpha);
            if (!lag)
                close_interval();
#pragma clang loop unroll(disable)
            for (int k = 1; k < n; ++k) {
                if (MASKED && ((k + 1) & 31) == 0)
                    walk_window(k + 1);
                s_half8(kaddr_of(k), qf, s, issue_loads(k));
                if (lag)
                    close_interval();
                causal_hide(k, s);
                pv_half8<MASKED, true, true>(vaddr_of(k - 1), o, pw, s, m, l, alpha, masked_vh(k));
                rescale(o, alpha);
                if (!lag)
                    close_interval();
            }
            if (lag)
                close_interval();
        }
        load_gates();                                    // the last context half covers the latency
        if (!MASKED || n > 0) {
            pv_half8<MASKED, true, false>(vaddr_of(n - 1), o, pw, s, m, l, alpha, 0u);
            if (!lag)
                close_interval();
        }
        epilogue();                                      // (masked, nothing visible: O and l stay zero)
    }
}

// ---------------------------------------------------------------------------
// Attention weights: bf16 [S][Hq][T], weight[i][h][j] = bf16(exp2((s_ij -
// m_ih) log2(e)/16) / l_ih) with s the bf16-rounded score and (m, l) the
// reference max and row sum the attention pass recorded; hidden keys give 0.
// Every element is written (zeros for tiles past a row block's diagonal and
// for tiles the mask hides from the whole block).
// grid (ceil(S/64), Hkv * n_hg, key splits), 512 threads, the attention kernel's work
// split: wave w takes query head 4 hg + (w & 3) of the block's KV head (idle
// past the group) and rows r0 + 32 (w >> 2) .. +31.  The eight waves stage
// each key tile once in LDS (the prepared tiles already have the LDS layout;
// the next tile's bytes wait in registers while the current one is used).
// The weight stores bound the kernel: each wave stages WT_GROUP tiles of its
// 32 rows and writes them as whole 128-byte row segments.
// ---------------------------------------------------------------------------
constexpr int WT_GROUP = 2;                         // tiles per staged group
constexpr int WT_ROW = WT_GROUP * KT * 2 + 16;       // staging bytes per row (padded)
constexpr int WT_SMEM = 2 * TILE_BYTES + 8 * 32 * WT_ROW;

template <int MODE>   // 0 causal, 1 masked (causal and mask), 2 bidirectional
__global__ __launch_bounds__(512) void attn_weights(AttnParams p, uint16_t *wout)
{
    __shared__ __attribute__((aligned(16))) char smem[WT_SMEM];
    __shared__ __align__(16) float wq1[D];
    __shared__ __align__(16) uint32_t wbits[MODE == 1 ? 2 : 1][QW];   // masked: a staged tile's row words
    fill_wq1(wq1, p.wq);
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hw = wave & 3, blk = wave >> 2;
    // Workgroups go to the eight XCDs in turn (linear id mod 8), each XCD with
    // its own L2.  Renumber so that XCD x takes the x-th eighth of the work,
    // ordered row block fastest: its blocks share a KV head and so its key tiles.
    int bx, by, bz;
    {
        const unsigned nb = gridDim.x * gridDim.y * gridDim.z, per = nb / 8;
        const unsigned b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
        const unsigned wk = (b < per * 8) ? (b % 8) * per + b / 8 : b;
        bx = (int)(wk % gridDim.x);
        by = (int)((wk / gridDim.x) % gridDim.y);
        bz = (int)(wk / (gridDim.x * gridDim.y));
    }
    const int kvh = by / p.n_hg, hg = by - kvh * p.n_hg;
    const int hq = 4 * hg + hw;                          // head within the KV group
    const bool active = hq < p.G;
    const int h = kvh * p.G + (active ? hq : 0);
    const int j = lane & 31, hh = lane >> 5;
    const int R0 = bx * QW;                              // the block's first row
    const int r0 = R0 + QB * blk;                        // this wave's rows r0 .. r0 + 31
    char *stage = smem + 2 * TILE_BYTES + wave * 32 * WT_ROW;

    uint4 qf[16];
    load_queries1(p, r0, h, lane, qf, wq1);
    const int rc = min(r0 + j, p.S - 1);
    const float m = p.ml[((size_t)rc * p.Hq + h) * 2];
    const float lsum = p.ml[((size_t)rc * p.Hq + h) * 2 + 1];
    const float nb = (m == -INFINITY) ? 0.0f : m * -SCALE_LOG2;
    const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
    const int P0 = p.q_base + R0;                        // a multiple of 64
    const int ntiles = (p.T + KT - 1) / KT;
    const int nvis = (MODE == 2 ? p.T - 1 : min(P0 + QW - 1, p.T - 1)) / KT + 1;   // the block's tiles
    const int diag = (P0 + QB * blk) / KT;               // this wave's diagonal tile
    const uint32_t diag_vis = (j == 31) ? 0xffffffffu : ((2u << j) - 1u);
    const FragOffsets fo = frag_offsets(j, hh);
    const bool vec = (p.T & 7) == 0;                     // 16-byte stores stay aligned
    const char *ktiles = reinterpret_cast<const char *>(p.kp + (size_t)kvh * (p.Tpad / KT) * (KT * D));

    // Key range: blockIdx.z takes groups [g_begin, g_begin + ng) of WT_GROUP
    // tiles, walked from a block-dependent starting group so that blocks
    // writing at the same time spread over the address space.
    const int ngroups_all = (ntiles + WT_GROUP - 1) / WT_GROUP;
    const int gper = (ngroups_all + gridDim.z - 1) / gridDim.z;
    const int g_begin = bz * gper;
    const int ng = max(min(gper, ngroups_all - g_begin), 0);
    const int rot = (ng > 0) ? (int)(((unsigned)bx * 5u + (unsigned)by * 3u) % (unsigned)ng) : 0;
    const int nq = ng * WT_GROUP;                        // walk positions
    auto tile_of = [&](int q) {
        int gg = q / WT_GROUP + rot;
        gg = gg >= ng ? gg - ng : gg;
        return (g_begin + gg) * WT_GROUP + q % WT_GROUP;
    };
    // Tiles the block computes: up to its diagonal, and (masked) visible to some row.
    auto computed = [&](int t) {
        return t < nvis && (MODE != 1 || p.tilevis[(size_t)(R0 / QW) * p.W + t] != 0);
    };
    auto next_computed = [&](int q) {
        for (++q; q < nq; ++q)
            if (computed(tile_of(q)))
                return q;
        return nq;
    };
    // Key tiles move global -> LDS with copies (two buffers, the next computed
    // tile in flight while the current one is used); masked, wave 0 also
    // copies the 64 rows' visibility words of the tile.  The vector memory
    // counter counts copies and stores together and retires them in order, so
    // a wait for a copy covers the stores issued before it, never those after:
    // the wait before a tile's barrier leaves the stores issued since its copy
    // (a whole group's four, when they were issued unconditionally) in flight.
    const uint32_t smem_base = lds_addr(smem);
    const uint32_t voff = (uint32_t)(wave * 2048 + lane * 16);
    auto stage_tile = [&](int t, int b) {
        const char *src = ktiles + (size_t)__builtin_amdgcn_readfirstlane(t) * TILE_BYTES;
        const uint32_t m0 =
            (uint32_t)__builtin_amdgcn_readfirstlane((int)(smem_base + TILE_BYTES * b + wave * 2048));
        dma16<0, true>(src, voff, m0);
        dma16<1024, true>(src, voff, m0);
        if (MODE == 1 && wave == 0)                      // row R0 + lane < bstride (pad rows hold zero words)
            dma4(p.bits, (uint32_t)(((size_t)__builtin_amdgcn_readfirstlane(t) * p.bstride + R0 + lane) * 4),
                 lds_addr(&wbits[b][0]));
    };
    int qnext = next_computed(-1);
    int nbuf = 0;
    if (qnext < nq)
        stage_tile(tile_of(qnext), 0);
    int stores_since = 0;                                // unconditional stores issued since the last copy
    // Write-out lane map: WT_LPR lanes per row, 16 bytes (8 keys) each.
    constexpr int WT_LPR = WT_GROUP * KT * 2 / 16, WT_RPI = 64 / WT_LPR;
    const int wr = lane / WT_LPR, wc = lane % WT_LPR;
    for (int gq = 0; gq < ng; ++gq) {
        const int t0 = tile_of(gq * WT_GROUP);
#pragma unroll
        for (int tl = 0; tl < WT_GROUP; ++tl) {
            const int q = gq * WT_GROUP + tl;
            const int t = t0 + tl;
            uint32_t w[16];
            if (q == qnext) {                            // block-uniform
                if (stores_since >= 4)
                    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();                         // the tile is in place; the other buffer is free
                const char *kb = smem + TILE_BYTES * nbuf;
                const int cur = nbuf;
                qnext = next_computed(q);
                nbuf ^= 1;
                if (qnext < nq) {
                    stage_tile(tile_of(qnext), nbuf);
                    stores_since = 0;
                }
                f32x16 s;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb + fo.k + 1024 * c);
                    const f32x16 z = {};
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, __builtin_bit_cast(bf16x8, qf[c]), c ? s : z,
                                                                0, 0, 0);
                }
                if (MODE == 1)
                    hide_all(s, wbits[cur][QB * blk + j] >> (4 * hh));
                else if (MODE == 0 && t >= diag)
                    hide_all(s, (t == diag ? diag_vis : 0u) >> (4 * hh));
                // rbf, not the inline-asm round_op: the scores come from the
                // MFMA builtin, and only a read the compiler sees gets the wait
                // states that reading a matrix-core result requires.
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    w[e] = f2bf(__builtin_amdgcn_exp2f(__builtin_fmaf(rbf(s[e]), SCALE_LOG2, nb)) * inv);
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    w[e] = 0u;
            }
            // Lane (j, hh) holds keys 8g + 4hh + r of row j: 8 bytes per g.
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint2 *>(stage + j * WT_ROW + (tl * KT + 8 * g + 4 * hh) * 2) =
                    make_uint2(w[4 * g] | (w[4 * g + 1] << 16), w[4 * g + 2] | (w[4 * g + 3] << 16));
        }
        // The wave reads back only what it wrote: its own LDS accesses stay in
        // order, and the compiler waits for the writes before these reads.
        // A group whose rows, keys and head all exist takes four unconditional
        // 16-byte streaming stores per lane; the others store what exists.
        const int key = t0 * KT + 8 * wc;
        const bool whole = active && vec && r0 + 32 <= p.S && (t0 + WT_GROUP) * KT <= p.T;   // wave-uniform
        if (whole) {
#pragma unroll
            for (int it = 0; it < 32 / WT_RPI; ++it) {
                const int rr = WT_RPI * it + wr;
                const uint4 v = *reinterpret_cast<const uint4 *>(stage + rr * WT_ROW + 16 * wc);
                uint16_t *dst = wout + ((size_t)(r0 + rr) * p.Hq + h) * p.T + key;
                __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(dst));
            }
            stores_since += 32 / WT_RPI;
        } else {
#pragma unroll
            for (int it = 0; it < 32 / WT_RPI; ++it) {
                const int rr = WT_RPI * it + wr;
                const int row = r0 + rr;
                const uint4 v = *reinterpret_cast<const uint4 *>(stage + rr * WT_ROW + 16 * wc);
                if (!active || row >= p.S || key >= p.T)
                    continue;
                uint16_t *dst = wout + ((size_t)row * p.Hq + h) * p.T + key;
                if (vec) {
                    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(dst));
                } else {
                    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (key + q < p.T)
                            dst[q] = (uint16_t)(words[q >> 1] >> (16 * (q & 1)));
                }
            }
            stores_since = 0;                            // count unknown: the next wait takes them all
        }
    }
}

// ---------------------------------------------------------------------------
// Calibration: the matrix-core rate this device sustains under its power
// limit.  One workgroup per compute unit, one wave per SIMD, back-to-back
// v_mfma_f32_32x32x16_bf16 on four independent accumulators with operands
// drawn from a xorshift generator (uniform in [-1, 1), i.e. every bit of the
// bf16 operands toggles like real data).  Each workgroup records its shader
// cycles (s_memtime) and 100 MHz ticks (s_memrealtime) over the loop.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mfma_clock_probe(int iters, long long *rec, float *sink)
{
    f32x16 acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[m][e] = 0.0f;
    bf16x8 a[4], b[4];
    uint32_t x = 2463534242u ^ (threadIdx.x * 7919u + blockIdx.x * 104729u);
    auto next = [&]() {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        return (float)(x & 0xffffu) * (1.0f / 32768.0f) - 1.0f;
    };
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[m][e] = (__bf16)next();
            b[m][e] = (__bf16)next();
        }
    const long long c0 = clock64(), r0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(m >> 2) & 3], b[m & 3], acc[m & 3], 0, 0, 0);
    }
    const long long c1 = clock64(), r1 = wall_clock64();
    float sum = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            sum += acc[m][e];
    sink[blockIdx.x * 256 + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        rec[2 * blockIdx.x] = c1 - c0;
        rec[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the prepared keys and
// transposed values of one call, in the workspace's tile layout.  Every device
// the library runs on holds its own copy until the process ends.  On the host
// the array's name is only a stand-in for the symbol, never a device address:
// host code uses the per-device address noalloc_scratch() returns.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint16_t scratch[kNoallocScratchBytes / sizeof(uint16_t)];

hipError_t noalloc_scratch(int device, uint16_t **ptr)
{
    static std::mutex mu;
    static uint16_t *addr[kNoallocMaxDevices] = {};
    if (device < 0 || device >= kNoallocMaxDevices || !ptr)
        return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void *a = nullptr;
        const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !a)
            return e != hipSuccess ? e : hipErrorInvalidSymbol;
        addr[device] = static_cast<uint16_t *>(a);
    }
    *ptr = addr[device];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_kv_prologue(const KvPrologueParams &p, int ntiles, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_prologue<false>, dim3(ntiles, p.Hkv), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_kv_prologue_fp8(const KvPrologueParams &p, int ntiles, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_prologue<true>, dim3(ntiles, p.Hkv), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_kv_widen(const KvWidenParams &p, int ntiles, int Hkv, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_widen, dim3(ntiles, Hkv), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mask_pack(const MaskPackParams &p, int nrb, hipStream_t stream)
{
    hipLaunchKernelGGL(mask_pack, dim3((p.W + 31) / 32, nrb), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnParams &p, AttnMode mode, hipStream_t stream)
{
    const int nblocks = p.n_wg;
    switch (mode) {
    case AttnMode::Masked:
        hipLaunchKernelGGL((attn_fwd8<true, false, false>), dim3(nblocks), dim3(ATHREADS8), 0, stream, p);
        break;
    case AttnMode::Bidirectional:
        hipLaunchKernelGGL((attn_fwd8<false, true, false>), dim3(nblocks), dim3(ATHREADS8), 0, stream, p);
        break;
    case AttnMode::SharedPrefix:
        hipLaunchKernelGGL((attn_fwd8<false, false, true>), dim3(nblocks), dim3(ATHREADS8), 0, stream, p);
        break;
    default:
        hipLaunchKernelGGL((attn_fwd8<false, false, false>), dim3(nblocks), dim3(ATHREADS8), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_attn_weights(const AttnParams &p, AttnMode mode, uint16_t *weights, int num_cus,
                               hipStream_t stream)
{
    // Split the keys over blockIdx.z until there are about two workgroups per
    // compute unit (two fit its LDS), keeping at least 16 tiles per split.
    const int blocks = ((p.S + QW - 1) / QW) * p.Hkv * p.n_hg;
    const int groups = ((p.T + KT - 1) / KT + WT_GROUP - 1) / WT_GROUP;
    int nz = (2 * num_cus + blocks - 1) / blocks;
    nz = std::max(1, std::min(nz, groups / (16 / WT_GROUP)));
    const dim3 grid((p.S + QW - 1) / QW, p.Hkv * p.n_hg, nz);
    if (mode == AttnMode::Masked)
        hipLaunchKernelGGL(attn_weights<1>, grid, dim3(512), 0, stream, p, weights);
    else if (mode == AttnMode::Bidirectional)
        hipLaunchKernelGGL(attn_weights<2>, grid, dim3(512), 0, stream, p, weights);
    else
        hipLaunchKernelGGL(attn_weights<0>, grid, dim3(512), 0, stream, p, weights);
    return hipGetLastError();
}

hipError_t launch_mfma_clock_probe(int iters, int n_wg, long long *rec, float *sink, hipStream_t stream)
{
    hipLaunchKernelGGL(mfma_clock_probe, dim3(n_wg), dim3(256), 0, stream, iters, rec, sink);
    return hipGetLastError();
}

#ifdef ATTN_TEST_HOOKS
hipError_t launch_kp_unpack(const uint16_t *kp, int Tpad, int T, int Hkv, uint16_t *out, hipStream_t stream)
{
    hipLaunchKernelGGL(kp_unpack, dim3((T + KT - 1) / KT, Hkv), dim3(256), 0, stream, kp, Tpad, T, out);
    return hipGetLastError();
}

hipError_t launch_q_prologue_debug(const AttnParams &p, uint16_t *qp, hipStream_t stream)
{
    hipLaunchKernelGGL(q_prologue_debug, dim3((p.S + 63) / 64, (p.Hq + 3) / 4), dim3(256), 0,
                       stream, p, qp);
    return hipGetLastError();
}

hipError_t launch_fp8_encode_debug(const float *x, const float *sc, float *q, uint8_t *codes, int64_t n,
                                   hipStream_t stream)
{
    hipLaunchKernelGGL(fp8_encode_debug, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, sc, q, codes,
                       n);
    return hipGetLastError();
}
#endif  // ATTN_TEST_HOOKS

}  // namespace ga
