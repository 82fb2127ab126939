// kernels.h -- parameters and launchers shared by kernels.hip and abi.cpp
// (internal to libgatedattn.so; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

struct KvPrologueParams {
    const uint16_t *k;        // [T][Hkv][256]
    const uint16_t *v;        // [T][Hkv][256]
    const uint16_t *wk;       // [256]
    const float *cos_tab;     // [n_pos][32]
    const float *sin_tab;     // [n_pos][32]
    uint16_t *kp;             // [Hkv][Tpad/32] tiles of 32 keys, chunk-major
    uint16_t *vt;             // [Hkv][Tpad/32] tiles of V^T, chunk-major
    int T, Hkv, Tpad;
    int tile0;                // first tile written (grid x = tile - tile0)
    int k_row0;               // position of row 0 of k and v
    float eps;
    // Packed batch (else null): tile_seg[x] = sequence of prepared tile x;
    // seg[4 s ..] = {length, first row in k/v, first prepared tile, position
    // of its first key} (the position is 0 but for the branches of a shared
    // prefix, which continue from the prefix's length).
    const int *tile_seg;
    const int *seg;
    // fp8 cache rows (kv_prologue<true> only): codes [Hkv][Tpad][256] and one
    // fp32 scale per row [Hkv][Tpad], keys then values; rows = positions.
    uint8_t *k8, *v8;
    float *k8s, *v8s;
};
struct KvWidenParams {
    const uint8_t *k8, *v8;   // fp8 cache rows [Hkv][Tpad][256]
    const float *k8s, *v8s;   // their scales [Hkv][Tpad]
    uint16_t *kp;             // [Hkv][Tpad/32] tiles of 32 keys, chunk-major
    uint16_t *vt;             // [Hkv][Tpad/32] tiles of V^T, chunk-major
    int T, Tpad;              // rows 0..T-1 are widened; tiles past them get zeros
};

struct MaskPackParams {
    const uint8_t *mask;      // [S][S]
    uint32_t *bits;           // [W][bstride]: key word major, rows contiguous
    uint8_t *tilevis;         // [nrb][W]
    int S, W;
    int bstride;              // rows per key word: S rounded up to 64 (pad rows 0)
    int vec16;                // mask rows may be read 16 bytes at a time
};

struct AttnParams {
    const uint16_t *qg;       // [S][Hq][2][256]
    const uint16_t *kp;       // [Hkv][Tpad/32] tiles of 32 keys, chunk-major
    const uint16_t *vt;       // [Hkv][Tpad/32] tiles of V^T, chunk-major
    const uint16_t *wq;       // [256]
    const float *cos_tab;     // [n_pos][32]
    const float *sin_tab;     // [n_pos][32]
    const uint32_t *bits;     // [W][bstride] (masked only; MaskPackParams)
    const uint8_t *tilevis;   // [nrb][W] (masked only)
    uint16_t *out;            // [S][Hq][256]
    int S, T, q_base;
    int Hq, Hkv, G, n_hg, nrb, Tpad, W;
    int bstride;              // masked only: rows per key word of bits
    int n_wg;                 // attention workgroups (<= work items)
    float eps;
    // Packed batch (else null): pairs[2 i ..] = {sequence, row block} of the
    // i-th (64-row block) in walk order, nrb = their count; seg as in
    // KvPrologueParams.  Each sequence is a causal pass at positions 0..len-1,
    // or (attn_fwd8_shared) a branch at positions pos0..pos0+len-1 over the
    // shared prefix's keys 0..pos0-1 (tiles of ckp / cvt) and its own.
    const int *pairs;
    const int *seg;
    // Optional (else null): per (row, query head) the softmax's final
    // reference max (raw score units) and row sum, [S][Hq][2] fp32.
    float *ml;
    // Optional (else null: the snake order of schedule.h): the host's table of
    // work items per workgroup (sched_plan), n_wg + 1 offsets then entries.
    const int *sched;
    // attn_fwd8_shared only (else null): the shared prefix's prepared key
    // and transposed value tiles (the caller's cache, Tpad as above).
    const uint16_t *ckp, *cvt;
};

constexpr int kRowsPerBlock = 64;
constexpr int kKeysPerTile = 32;
constexpr int kHeadsPerBlock = 4;

// Scratch of the allocation-free entry point: prepared keys and transposed
// values of one call (2 x Hkv x round_up(S, 64) x 256 bf16), one fixed array
// per device (kernels.hip).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
constexpr int kNoallocMaxDevices = 64;
// The device address of this device's scratch array (the current device must
// be `device`); looked up once per device with hipGetSymbolAddress.
hipError_t noalloc_scratch(int device, uint16_t **ptr);

hipError_t launch_kv_prologue(const KvPrologueParams &p, int ntiles, hipStream_t stream);
hipError_t launch_kv_prologue_fp8(const KvPrologueParams &p, int ntiles, hipStream_t stream);
hipError_t launch_kv_widen(const KvWidenParams &p, int ntiles, int Hkv, hipStream_t stream);
hipError_t launch_mask_pack(const MaskPackParams &p, int nrb, hipStream_t stream);
enum class AttnMode { Causal, Masked, Bidirectional, SharedPrefix };
hipError_t launch_attention(const AttnParams &p, AttnMode mode, hipStream_t stream);
hipError_t launch_attn_weights(const AttnParams &p, AttnMode mode, uint16_t *weights, int num_cus,
                               hipStream_t stream);
hipError_t launch_mfma_clock_probe(int iters, int n_wg, long long *rec, float *sink, hipStream_t stream);
#ifdef ATTN_TEST_HOOKS
// Test build only: prepared keys / queries back in plain layouts; the fp8
// cache writer's division and encode on single values.
hipError_t launch_kp_unpack(const uint16_t *kp, int Tpad, int T, int Hkv, uint16_t *out, hipStream_t stream);
hipError_t launch_q_prologue_debug(const AttnParams &p, uint16_t *qp, hipStream_t stream);
hipError_t launch_fp8_encode_debug(const float *x, const float *sc, float *q, uint8_t *codes, int64_t n,
                                   hipStream_t stream);
#endif

}  // namespace ga
