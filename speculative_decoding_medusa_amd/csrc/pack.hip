// Packing of bf16 weight matrices into the MFMA fragment order that
// skinny_mfma_kernel streams: row r, column k of a packed matrix with K
// columns and NRB = ceil(rows / 16) blocks of 16 rows sits at element
//     ((k / 32) * NRB + r / 16) * 512 + ((k % 32) / 8 * 16 + r % 16) * 8 + k % 8,
// i.e. every 16 x 32 tile is one contiguous 1 KB fragment in the lane order of
// the A operand of v_mfma_f32_16x16x32_bf16, and the fragments of one 32-wide
// step of the contraction are contiguous over all row blocks (k-step major):
// while the waves of a product advance through the contraction together, the
// whole GPU reads one narrow, contiguous window of the matrix, which the HBM
// serves better than one stream per row block (measured 3-12% faster on the
// 7B lm_head and decoder projections).  A packed matrix of `rows` rows holds
// NRB * 16 * K elements; several row-major matrices can be packed into one,
// stacked along the rows (each at its row offset) or interleaved in blocks of
// 16 rows (block j of matrix m at packed block j * n + m, for n matrices).
#include <algorithm>

#include "common.hpp"
#include "skinny_mfma.hpp"

namespace medusa {

size_t packed_elems(int rows, int K) { return (size_t)((rows + PACK_ROWS - 1) / PACK_ROWS) * PACK_ROWS * K; }

// One thread per 8-element piece: reads src row-major (coalesced), writes the
// piece to its fragment slot.  Source row i goes to packed row
// dst_row0 + (i / 16) * 16 * inter + i % 16 of a packed matrix of nrb row
// blocks.  Rows i >= rows (the padding of the last fragment row block,
// written only when a plain call ends the matrix) get zeros.
__global__ __launch_bounds__(256) void pack_rows_kernel(const bf16_t* __restrict__ src, int rows, int rows_out, int K,
                                                        bf16_t* __restrict__ dst, int dst_row0, int inter, int nrb) {
    const size_t per_row = (size_t)K / 8;
    const size_t total = (size_t)rows_out * per_row;
    for (size_t p = blockIdx.x * (size_t)blockDim.x + threadIdx.x; p < total; p += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(p / per_row);
        const int k8 = (int)(p - (size_t)i * per_row);
        const u32x4 v = i < rows ? *(const u32x4*)(src + (size_t)i * K + (size_t)k8 * 8) : (u32x4){0u, 0u, 0u, 0u};
        const int r = dst_row0 + (i / PACK_ROWS) * PACK_ROWS * inter + i % PACK_ROWS;
        const size_t frag = (size_t)(k8 / 4) * nrb + r / PACK_ROWS;
        *(u32x4*)(dst + frag * PACK_FRAG + ((k8 & 3) * PACK_ROWS + r % PACK_ROWS) * 8) = v;
    }
}

void launch_pack_rows(const bf16_t* src, int rows, int K, bf16_t* dst, int dst_row0, int dst_rows, int inter,
                      hipStream_t s) {
    const int end = dst_row0 + rows;
    const int rows_out = inter == 1 && end == dst_rows ? (int)(packed_elems(dst_rows, K) / K) - dst_row0 : rows;
    const size_t total = (size_t)rows_out * (K / 8);
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 8192);
    const int nrb = (dst_rows + PACK_ROWS - 1) / PACK_ROWS;
    MEDUSA_LAUNCH("pack_rows", pack_rows_kernel, dim3(blocks), dim3(256), 0, s, src, rows, rows_out, K, dst, dst_row0, inter,
                  nrb);
}

}  // namespace medusa
