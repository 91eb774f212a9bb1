// LDS tile machinery shared by the bf16 attention kernels (forward and backward): a 64x64
// bf16 tile staged row-major in LDS by direct-to-LDS buffer loads, with an XOR swizzle of
// its 16-byte chunks, read back as matrix-core operands either by rows (ds_read_b128) or
// transposed (ds_read_b64_tr_b16).
#pragma once

#include "device.h"

namespace s3d {
namespace tl {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int TILE_BYTES = TILE * 128;           // one bf16 64x64 tile

// Physical 16-byte slot of logical chunk `chunk` in tile row `row`.  The XOR key uses
// row bits 0-3 so that, with 64 LDS banks served 16 lanes (b128) or 32 lanes (b64) per
// pass, both the K-operand reads (16 rows, one chunk each) and the transposing V reads
// (4 rows, 4 chunks each) touch every bank at most once per pass.
__device__ __forceinline__ int swz_key(int row) {
    return (((row & 2) << 1) | ((row >> 2) & 3)) ^ ((row & 1) << 1);
}
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ swz_key(row); }

// Word 3 of a raw buffer resource on gfx9-class parts (32-bit data format, no swizzle).
constexpr int BUF_RSRC_WORD3 = 0x00020000;
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int WAITCNT_VM0_LGKM0 = 0x0070;        // vmcnt(0) lgkmcnt(0)
constexpr int WAITCNT_LGKM0 = 0xC07F;            // lgkmcnt(0) only
// Scheduling-barrier mask: ALU, VALU, SALU, matrix, LDS and transcendental instructions may
// move across it, vector-memory instructions may not.
constexpr int SCHED_ALLOW_ALL_BUT_VMEM = 0x1 | 0x2 | 0x4 | 0x8 | 0x80 | 0x100 | 0x200 | 0x400;

// A byte offset past every per-head buffer: buffer loads there return zeros.
constexpr unsigned OOB_OFFSET = 0x80000000u;

// 16 bytes per lane from buffer `rs` at byte offset voff + soff into LDS at
// lds_base + 16 * lane.
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t rs, lds_u8* lds_base, unsigned voff,
                                        unsigned soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}

// Per-lane LDS byte offsets of the two operand reads, for a lane with column index qc
// (lane % 32) and group g (lane / 32):
//  - by rows: rows qc and qc + 32 (4 KiB further, same swizzle key), 16-dim step st,
//    dims 16 st + 8 g .. +8: the A operand of X * Y^T with X in LDS;
//  - transposed (ds_read_b64_tr_b16): lane j of each 16-lane group points at
//    X[16 ks + 8 half + 4 g + j/4][32 cb + 16 ((lane/16) % 2) + 4 (j % 4)]; rows for
//    different ks differ by multiples of 16, which leave the swizzle key unchanged.  This
//    gives the A operand X^T (dims x rows) whose k order matches the rows a lane holds in
//    a 32x32 accumulator (8 (r/4) + 4 g + r % 4), so an accumulator converted to bf16 is
//    directly the B operand.
struct TileOffsets {
    int row[4];        // by rows, per 16-dim step
    int tr[2][2];      // transposed, [column block][half]
    __device__ __forceinline__ void init(int lane) {
        const int qc = lane & 31, g = lane >> 5;
#pragma unroll
        for (int st = 0; st < 4; ++st) row[st] = qc * 128 + swz(qc, 2 * st + g) * 16;
        const int r0 = 4 * g + ((lane & 15) >> 2);
        const int cchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int sub = (lane & 1) * 8;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int r = r0 + 8 * hf;
                tr[cb][hf] = r * 128 + swz(r, 4 * cb + cchunk) * 16 + sub;
            }
    }
};

// A operand rows qc (a0) and qc + 32 (a1), dims 16 st + 8 g .. +8, of the tile at t
__device__ __forceinline__ void read_rows(const unsigned char* t, const TileOffsets& o, int st,
                                          bf16x8& a0, bf16x8& a1) {
    a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t + o.row[st]));
    a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t + o.row[st] + 4096));
}

// A operand X^T for k-step ks (16 rows of the tile): column block 0 (a0) and 1 (a1)
__device__ __forceinline__ void read_tr(const unsigned char* t, const TileOffsets& o, int ks,
                                        bf16x8& a0, bf16x8& a1) {
    const lds_u8* lb = (const lds_u8*)t;
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lb + o.tr[0][0] + ks * 2048));
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lb + o.tr[0][1] + ks * 2048));
    const v4i16 y0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lb + o.tr[1][0] + ks * 2048));
    const v4i16 y1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lb + o.tr[1][1] + ks * 2048));
    a0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    a1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B operand for k-step ks from a pair of 32x32 accumulators (rows 0-31 in x0, 32-63 in
// x1), each value mapped by f (e.g. a probability or a gradient) and rounded to bf16.
template <typename F>
__device__ __forceinline__ bf16x8 acc_to_b(const f32x16& x0, const f32x16& x1, int ks, F&& f) {
    const f32x16& xp = ks < 2 ? x0 : x1;
    const int j0 = 2 * (ks & 1);
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (__bf16)f(xp[4 * j0 + i], 4 * j0 + i, ks < 2 ? 0 : 1);
    return b;
}

}  // namespace tl
}  // namespace s3d
