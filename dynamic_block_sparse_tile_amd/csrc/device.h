// Device-side types and helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace s3d {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 64;   // rows per tile; also the head dimension
constexpr int HD = 64;
constexpr int NXCD = 8;    // MI355X: 8 accelerator complex dies, each with its own L2

// A token sequence as the kernels see it (see sparse3d_layout).
struct Lay {
    int S, N, P, nsp;      // frames, valid tokens per frame, stride, specials
};

// bf16 bits <-> fp32.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
// Round-to-nearest-even fp32 -> bf16 of two values, packed low|high (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// Workgroups are dispatched round-robin over the XCDs (workgroup i runs on XCD i % 8).
// Renumber them so that each XCD receives one contiguous range of logical work items:
// neighbouring items (which read overlapping key tiles) then share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int per = nblocks / NXCD, rem = nblocks % NXCD;
    const int xcd = bid % NXCD, slot = bid / NXCD;
    // XCDs [0, rem) own per+1 items, the rest own per.
    const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return base + slot;
}

// Work item of an attention workgroup.  Query tiles come in groups G = (head h, in-frame
// tile j), the S query tiles (one per frame) at the same position j of one head; the tiles
// of a group select overlapping key tiles (the same scene content seen in every frame).
// Each XCD receives one contiguous range of workgroups (xcd_remap) and its range holds
// whole groups, G = x, x + 8, x + 16, ... for XCD x, in increasing order.  So at any time
// one group runs per XCD (its key tiles share that XCD's L2) and all XCDs work on
// neighbouring groups of the same head (whose K and V then share the last-level cache),
// instead of each XCD streaming a different head.
// (Frame attention reads only the query's own frame, so there the plain order, frame by
// frame, is the one that shares key tiles: `grouped` = false.)
__device__ __forceinline__ void attn_work_item(int bid, int nblocks, int S, int tpf, int heads,
                                               int& h, int& tq, bool grouped = true) {
    const int logical = xcd_remap(bid, nblocks);
    if (!grouped) {
        const int tqs = S * tpf;
        h = logical / tqs;
        tq = logical - h * tqs;
        return;
    }
    int rank = logical / S;
    const int s = logical - rank * S;
    int G = rank;
    const int ng = heads * tpf;
    for (int x = 0; x < NXCD; ++x) {
        const int c = (ng - x + NXCD - 1) / NXCD;   // groups with G % NXCD == x
        if (rank < c) {
            G = x + NXCD * rank;
            break;
        }
        rank -= c;
    }
    h = G / tpf;
    tq = s * tpf + (G - h * tpf);
}

// Member-row range [lo, hi) of key tile t inside its 64 rows (patch tokens only).
__device__ __forceinline__ void member_range(const Lay& L, int t, int& lo, int& hi) {
    const int tpf = L.P / TILE;
    const int j0 = (t % tpf) * TILE;
    lo = max(0, L.nsp - j0);
    hi = min(TILE, L.N - j0);
    if (hi < lo) hi = lo;
}
// Valid-query (or dense key) row count of tile t: rows with in-frame position < N.
__device__ __forceinline__ int valid_rows(const Lay& L, int t) {
    const int tpf = L.P / TILE;
    const int j0 = (t % tpf) * TILE;
    return max(0, min(TILE, L.N - j0));
}

__device__ __forceinline__ uint64_t range_mask(int lo, int hi) {
    const uint64_t upto_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
    const uint64_t below_lo = lo >= 64 ? ~0ull : ((1ull << lo) - 1ull);
    return upto_hi & ~below_lo;
}

}  // namespace s3d
