// Repack of the caller's Q4_K blobs into the library's device layout.
//
// Same 144 bytes per 256 weights, reordered so that one 16-byte load per lane
// delivers MFMA-ready quant fragments:
//   matrix -> [expert][row group of 16 rows][super-block b][2304 bytes]
//   2304 = 2048 quant bytes + 256 header bytes.
//   quant part: [half p = 0,1][lane group g = 0..3][row n = 0..15][16 bytes]
//     the 16 bytes are quant bytes 64p + 8g .. +8 (chunk 2p, this lane's 8
//     columns of sub-blocks 4p and 4p+1) followed by quant bytes
//     64p + 32 + 8g .. +8 (chunk 2p+1, sub-blocks 4p+2 and 4p+3);
//     lane l = n + 16g of a wave reads byte offset p*1024 + 16*l.
//   header part: row n's original bytes 0..15 (d, dmin, 12 scale bytes) at 16n.
// Gate and up share one matrix of 2I rows: row group rg holds gate rows
// 8rg .. 8rg+7 as n = 0..7 and up rows 8rg .. 8rg+7 as n = 8..15, so each
// wave's 16 output columns pair a gate row with its up row (SwiGLU in the
// epilogue). Down rows map to row group r/16, n = r%16.
#pragma once
#include "common.hpp"

namespace moe {

// One thread per (source row, super-block). kind 0 = gate, 1 = up, 2 = down.
__global__ void repack_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int E, int rows,
                              int nsb, int kind) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)E * rows * nsb;
    if (i >= total) return;
    const int b = (int)(i % nsb);
    const long er = i / nsb;
    const int r = (int)(er % rows);
    const int e = (int)(er / rows);
    int rg, n, ngroups;
    if (kind == 2) {
        rg = r / kRowGroup;
        n = r % kRowGroup;
        ngroups = rows / kRowGroup;
    } else {
        rg = r / 8;
        n = (r % 8) + (kind == 1 ? 8 : 0);
        ngroups = rows / 8;
    }
    const uint8_t *s = src + (size_t)i * kQ4Bytes;
    uint8_t *d = dst + ((size_t)((size_t)e * ngroups + rg) * nsb + b) * kGroupSbBytes;
    const u32x4 hdr = *(const u32x4 *)s;
    *(u32x4 *)(d + kGroupQsBytes + 16 * n) = hdr;
    const uint8_t *qs = s + 16;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2 a = *(const u32x2 *)(qs + 64 * p + 8 * g);
            const u32x2 c = *(const u32x2 *)(qs + 64 * p + 32 + 8 * g);
            u32x4 v = {a.x, a.y, c.x, c.y};
            *(u32x4 *)(d + p * 1024 + (g * 16 + n) * 16) = v;
        }
    }
}

}  // namespace moe
