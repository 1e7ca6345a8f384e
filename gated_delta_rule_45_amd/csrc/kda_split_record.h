// Per-chunk record of the two-pass forward (written by its prep kernel, or by the backward's prep
// kernel for the backward's forward pass; read by the forward's scans) and its store helpers.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ------------------------------------------------------------------ record --
template <typename IO, int DK, int C>
struct SplitRecord {
    static constexpr bool BF = IoTraits<IO>::kBf16;
    static constexpr int NSUB = C / 16;
    static constexpr int KT = DK / 16;
    static constexpr int NPAIR = (NSUB + 1) / 2;  // 32-wide token tile pairs
    static constexpr int FRAG_BYTES = BF ? 8 : 16;
    static constexpr int PAIR_BYTES = 2 * FRAG_BYTES;
    static constexpr int TILE_BYTES = 64 * PAIR_BYTES;  // one 16 x 32 operand tile
    static constexpr size_t oKt = 0;
    static constexpr size_t oQt = oKt + (size_t)NSUB * (KT / 2) * TILE_BYTES;
    static constexpr size_t oKbT = oQt + (size_t)NSUB * (KT / 2) * TILE_BYTES;
    // T and P are block lower triangular: row tile R keeps only its 32-wide column pairs
    // pp <= R / 2, stored row tile after row tile.  For even R the last pair's right 16 columns
    // lie above the diagonal, so that tile keeps only its left fragment (a half tile).
    static constexpr int HALF_BYTES = 64 * FRAG_BYTES;
    __host__ __device__ static constexpr bool tp_half(int R, int pp) { return R % 2 == 0 && 2 * pp == R; }
    __host__ __device__ static constexpr int tp_off(int R, int pp) {  // byte offset inside T or P
        int off = 0;
        for (int r = 0; r < R; ++r) off += (r / 2) * TILE_BYTES + (r % 2 == 0 ? HALF_BYTES : TILE_BYTES);
        return off + pp * TILE_BYTES;
    }
    static constexpr int TP_BYTES = (tp_off(NSUB, 0) + 1023) / 1024 * 1024;  // whole copy units
    static constexpr size_t oT = oKbT + (size_t)KT * NPAIR * TILE_BYTES;
    static constexpr size_t oP = oT + (size_t)TP_BYTES;
    static constexpr size_t oGam = oP + (size_t)TP_BYTES;
    static constexpr size_t kRaw = oGam + (size_t)DK * 4;
    static constexpr size_t kBytes = (kRaw + 1023) / 1024 * 1024;  // whole 1 KB copy units
    static_assert(KT % 2 == 0, "d_k must be a multiple of 32");
};

// store one lane's two 16-wide fragments of a 16 x 32 tile.  Record writes are nontemporal:
// the scan reads them only after this kernel ends, and dirty record lines left in L2 slowed the
// scan's first loads (prefill call 222 -> 218 us with these stores nontemporal).
template <bool BF>
__device__ __forceinline__ void store_pair(char *tile, int lane, const Frag<BF> &a, const Frag<BF> &b) {
    if constexpr (BF) {
        const u32x4 w = {a.v.x, a.v.y, b.v.x, b.v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(tile + lane * 16));
    } else {
        const f32x4 x = {a.v.x, a.v.y, a.v.z, a.v.w}, y = {b.v.x, b.v.y, b.v.z, b.v.w};
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(tile + lane * 32));
        __builtin_nontemporal_store(y, reinterpret_cast<f32x4 *>(tile + lane * 32 + 16));
    }
}
// one lane's left fragment of a half tile
template <bool BF>
__device__ __forceinline__ void store_frag(char *tile, int lane, const Frag<BF> &a) {
    *reinterpret_cast<decltype(a.v) *>(tile + lane * (int)sizeof(a.v)) = a.v;
}

}  // namespace kda
